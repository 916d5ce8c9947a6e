// One-launch W4A16 routed-MoE decode of a single token on gfx950.
//
// Batch-1 decode reads every active weight once and does almost no
// arithmetic per byte ("Let's optimize Nemotron 3.5 Lightning - a worklog",
// Interlude), so the whole layer runs as ONE persistent launch whose waves
// stream the selected experts' 4-bit weights over the entire chip:
//
//   R  router:  workgroup e (< E) computes logit e (its four waves split the
//               row of W_g), the sigmoid score and the key score + bias, and
//               publishes them with a release increment of a counter.
//   S  select:  every wave waits for all E keys and runs the exact fp32
//               top-k itself (wave max, then the lowest index holding it).
//   U  up:      the K x I (slot, row) units are split evenly over all waves;
//               each wave first issues the loads of its up rows AND (waves
//               0..6) of its down rows, which do not depend on h, then
//               computes h = relu(W_up x)^2 for its rows into LDS.
//   P  publish: wave 7 of each workgroup, which holds no down rows and so has
//               no loads in flight, writes the workgroup's h rows out, waits
//               for its own stores, bumps per-slot counters, then waits for
//               the slots the workgroup's down rows need and stages them in
//               LDS.  (A wave cannot wait for its stores or a polled value
//               without also waiting for every load it has in flight.)
//   D  down:    waves 0..6 finish z = w * g * (W_down h) from the weights
//               already in registers and publish per-block counts.
//   C  combine: the wave completing a 64-row block sums z over the slots in
//               slot order (deterministic) and writes y32 and bf16 y.
//
// Cross-workgroup hand-offs: the few values that cross workgroups (keys,
// h, z) are written and read with device-coherent accesses (relaxed
// agent-scope atomics, i.e. sc1 loads and stores that bypass the per-XCD L2
// copies), each writer waits for its stores to complete before it bumps a
// counter, and readers spin on the counter.  This avoids agent-scope fences,
// which on a multi-XCD part write back or invalidate a whole L2.  Counter
// updates are aggregated per workgroup.  Every wait is bounded (about 0.1 s
// of wall clock); on expiry the kernel flags the workspace and carries on,
// so it always ends.  The last workgroup to leave zeroes the counters.
#pragma once

#include "q4moe_kernels.hpp"

// Phase marker for instrumented builds; expands to nothing in the library.
#ifndef Q4MOE_PHASE
#define Q4MOE_PHASE(i)
#endif

namespace q4moe {

// Values many workgroups read (the router keys, h) and the counters they
// poll are kept in kReplicas copies; workgroup b uses copy b % kReplicas,
// which is also its XCD (workgroups are dealt to the XCDs round-robin), so
// no single cache line or memory channel serves the whole chip.
constexpr int kReplicas = 8;

// Workspace control word indices of the fused decode.
enum : int {
    FW_EXIT = 3,     // workgroups finished
    FW_ROUTER = 8,   // [kReplicas]: keys published
    FW_UP = 16,      // [8 slots][kReplicas]: up rows published per slot
    FW_BLOCK = 80,   // [n_blocks]: down units published per 64-row block
};
constexpr int kFusedMaxBlocks = 64;  // H <= 4096
constexpr int kMaxWgUp = 512;        // up rows per workgroup (K * I / grid)
constexpr int kRowBlock = 64;
constexpr uint64_t kSpinTicks = 10000000ull;  // 0.1 s of the 100 MHz real-time counter

struct FusedArgs {
    int E, H, I, K;
    const float* wg;
    const float* bias;
    const uint16_t* x;
    const uint8_t* upc;
    const void* ups;
    const float* upg;
    const uint8_t* dnc;
    const void* dns;
    const float* dng;
    uint16_t* y;
    int32_t* ids_out;  // nullable
    float* w_out;      // nullable
    uint32_t* ctrl;
    float* keys;       // [kReplicas][E]
    float* scores;     // [kReplicas][E]
    int32_t* ids;      // [K]
    float* w;          // [K]
    float* h;          // [kReplicas][K][I]
    float* z;          // [K][H]
    float* y32;        // [H]
};

constexpr int kWaves = 8;  // waves per workgroup (one workgroup per CU)

// Device-coherent store / load of a value another workgroup reads / wrote.
__device__ __forceinline__ void put_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_coherent2(const float* p) {
    return __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have completed (and keep the compiler from
// moving memory accesses across this point).
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t load_counter(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by one lane: wait until *p >= target; false (and a flag) on expiry.
__device__ __noinline__ bool spin_until(uint32_t* p, uint32_t target, uint32_t* flags) {
    if (load_counter(p) >= target) return true;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (load_counter(p) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
            atomicOr(flags, 1u);
            return false;
        }
    }
    return true;
}


// Wave maximum of v (every lane receives it).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x128>(v));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

// Exact fp32 top-k of E <= 256 keys by one wave: expert e sits in lane
// e % 64, register e / 64.  Each round takes the wave maximum and then the
// lowest expert index holding it (ballot + find-first-set), so equal keys
// go to the lower index exactly as the definition says.  The ids and the
// renormalised gates go to this wave's LDS slots (read back per lane).
__device__ __forceinline__ void wave_topk(const FusedArgs& a, const float* s_keys, const float* s_scores,
                                          int* s_ids, float* s_w) {
    const int lane = threadIdx.x & 63;
    float key[4], sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        const bool live = e < a.E;
        key[q] = live ? s_keys[e] : -__builtin_inff();
        sc[q] = live ? s_scores[e] : 0.f;
    }
    float ssum = 0.f;
    for (int i = 0; i < a.K; ++i) {
        const float m = wave_max(fmaxf(fmaxf(key[0], key[1]), fmaxf(key[2], key[3])));
        int best = 0x7fffffff;
        float bs = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned long long hit = __ballot(key[q] == m);
            if (hit && best == 0x7fffffff) {
                const int l = (int)__builtin_ctzll(hit);
                best = l + 64 * q;
                bs = __shfl(sc[q], l, 64);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q == best) key[q] = -__builtin_inff();
        if (best >= a.E) {  // no finite key left (NaN keys): keep every read inside the bank
            best = 0;
            if (lane == 0) atomicOr(a.ctrl + CTRL_FLAGS, 2u);
        }
        if (lane == 0) {
            s_ids[i] = best;
            s_w[i] = bs;
        }
        ssum += bs;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < a.K) s_w[lane] = s_w[lane] / ssum;
    __builtin_amdgcn_wave_barrier();
}

// Workgroup e computes router logit e: its waves split the row of W_g.
__device__ __forceinline__ void router_wg(const FusedArgs& a, int e, float* s_part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nf4 = a.H / 4;
    const int lo = wave * nf4 / kWaves, hi = (wave + 1) * nf4 / kWaves;
    const float4* wr = reinterpret_cast<const float4*>(a.wg + (size_t)e * a.H);
    float acc = 0.f;
    for (int j = lo + lane; j < hi; j += 64) {
        const float4 wv = wr[j];
        const uint2 xb = *reinterpret_cast<const uint2*>(a.x + 4 * j);
        acc = __builtin_fmaf(wv.x, bf16_bits_to_f32(xb.x & 0xffffu), acc);
        acc = __builtin_fmaf(wv.y, bf16_bits_to_f32(xb.x >> 16), acc);
        acc = __builtin_fmaf(wv.z, bf16_bits_to_f32(xb.y & 0xffffu), acc);
        acc = __builtin_fmaf(wv.w, bf16_bits_to_f32(xb.y >> 16), acc);
    }
    acc = seg_sum<64>(acc);
    if (lane == 0) s_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x < kReplicas) {  // one replica per thread
        float l = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) l += s_part[v];
        const float s = 1.0f / (1.0f + expf(-l));
        const int rep = threadIdx.x;
        put_coherent(a.keys + rep * a.E + e, s + a.bias[e]);
        put_coherent(a.scores + rep * a.E + e, s);
        stores_done();
        atomicAdd(a.ctrl + FW_ROUTER + rep, 1u);
    }
}

// Thread 0 waits for a counter, then the whole workgroup proceeds.
__device__ __forceinline__ void wg_wait(uint32_t* p, uint32_t target, uint32_t* flags) {
    if (threadIdx.x == 0) spin_until(p, target, flags);
    compiler_fence();
    __syncthreads();
}

// Units of [0, total) owned by wave index `w` of `n` waves: [lo, hi).
__device__ __forceinline__ int share_lo(int total, int w, int n) { return (int)((long long)w * total / n); }

template <int FMT, int C, int C2>
__global__ __launch_bounds__(64 * kWaves, 1) void k_decode_fused(FusedArgs a) {
    constexpr int kMaxUp = 4;    // up passes (two rows each) whose loads are in flight together
    constexpr int kMaxDown = 10;  // down rows whose loads are in flight together
    __shared__ float s_part[kWaves];
    __shared__ int s_blocks[kWaves + 1];
    __shared__ float s_keys[256], s_scores[256];
    __shared__ int s_ids_all[kWaves][8];
    __shared__ float s_w_all[kWaves][8];
    __shared__ float s_h[2][4096];  // h of the (at most two) slots this workgroup's down rows use
    __shared__ float s_hrow[kMaxWgUp];  // this workgroup's up results, before they are published
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane >> 5, li = lane & 31;
    const int NW = gridDim.x * kWaves, gw = blockIdx.x * kWaves + wave;
    // down rows go to waves 0..kWaves-2; wave kWaves-1 is the control wave
    constexpr int kDownWaves = kWaves - 1;
    const bool ctl = wave == kWaves - 1;
    const int NWD = gridDim.x * kDownWaves, gwd = blockIdx.x * kDownWaves + (ctl ? 0 : wave);
    const int nchH = a.H / 32, nchI = a.I / 32;
    uint32_t* flags = a.ctrl + CTRL_FLAGS;
    const int rep = blockIdx.x % kReplicas;

    // activations of this lane's up chunks (independent of the routing)
    uint32_t xa[C][16];
    float xs[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = li * C + c;
        xs[c] = 0.f;
        if (ch < nchH) {
            uint32_t nat[16];
            load_x_chunk(a.x, ch, nat);
            if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
                for (int j = 0; j < 16; ++j) xa[c][j] = nat[j];
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d) int4_pair_order(nat + 4 * d, xa[c] + 4 * d);
                xs[c] = pair_sum_bf16(nat);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) xa[c][j] = 0u;
        }
    }

    Q4MOE_PHASE(0);
    // ---- R: router
    if ((int)blockIdx.x < a.E) router_wg(a, blockIdx.x, s_part);

    Q4MOE_PHASE(1);
    // ---- S: selection (every wave, from one copy of the keys per workgroup)
    wg_wait(a.ctrl + FW_ROUTER + rep, (uint32_t)a.E, flags);
    Q4MOE_PHASE(2);
    if ((int)threadIdx.x < a.E) {
        s_keys[threadIdx.x] = get_coherent(a.keys + rep * a.E + threadIdx.x);
        s_scores[threadIdx.x] = get_coherent(a.scores + rep * a.E + threadIdx.x);
    }
    __syncthreads();
    int* ids = s_ids_all[wave];
    float* wsel = s_w_all[wave];
    wave_topk(a, s_keys, s_scores, ids, wsel);
    if (gw == 0 && lane < a.K) {
        const int id = ids[lane];
        const float wv = wsel[lane];
        a.ids[lane] = id;
        a.w[lane] = wv;
        if (a.ids_out) a.ids_out[lane] = id;
        if (a.w_out) a.w_out[lane] = wv;
    }

    Q4MOE_PHASE(3);
    // ---- U: issue the up loads of this wave's rows, then its down loads
    // per-tensor scales of the selected experts (lane i holds slot i's)
    float gu_l = 1.0f, gd_l = 1.0f;
    if constexpr (FMT == FMT_NVFP4) {
        const int sl = lane < a.K ? lane : 0;
        gu_l = a.upg[ids[sl]];
        gd_l = a.dng[ids[sl]];
    }
    const int RU = a.K * a.I, RD = a.K * a.H;
    const int u0 = share_lo(RU, gw, NW), u1 = share_lo(RU, gw + 1, NW);
    const int d0 = ctl ? 0 : share_lo(RD, gwd, NWD), d1 = ctl ? 0 : share_lo(RD, gwd + 1, NWD);

    // A wave's units span at most two slots (its share is shorter than a
    // slot): slot(u) = us0 + (u >= ubnd).
    const int us0 = (u1 > u0 ? u0 : 0) / a.I, ubnd = (us0 + 1) * a.I;
    const int ds0 = (d1 > d0 ? d0 : 0) / a.H, dbnd = (ds0 + 1) * a.H;

    // Every lane issues every load (an invalid row or chunk reads a valid
    // address and is zeroed through its scale at compute time), so the loads
    // stay in issue order and each use waits only for its own data.
    uint4 qu[kMaxUp][C];
    uint32_t su[kMaxUp][C];
    auto issue_up = [&](int pbase) {
#pragma unroll
        for (int p = 0; p < kMaxUp; ++p) {
            int u = u0 + 2 * (pbase + p) + seg;
            if (u >= u1) u = u1 > u0 ? u0 : 0;
            const int slot = us0 + (u >= ubnd ? 1 : 0), r = u - slot * a.I;
            const size_t row = (size_t)ids[slot] * a.I + r;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int ch = min(li * C + c, nchH - 1);
                qu[p][c] = ldg16(a.upc + row * (a.H / 2) + ch * 16);
                if constexpr (FMT == FMT_NVFP4)
                    su[p][c] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.ups) +
                                                                 row * (a.H / 16) + ch * 2);
                else
                    su[p][c] = reinterpret_cast<const uint16_t*>(a.ups)[row * (a.H / 64) + (ch >> 1)];
            }
        }
    };

    uint4 qd[kMaxDown][C2];
    uint32_t sd[kMaxDown][C2];
    auto issue_down = [&](int dbase) {
#pragma unroll
        for (int p = 0; p < kMaxDown; ++p) {
            int d = d0 + dbase + p;
            if (d >= d1) d = d1 > d0 ? d0 : 0;
            const int slot = ds0 + (d >= dbnd ? 1 : 0), r = d - slot * a.H;
            const size_t row = (size_t)ids[slot] * a.H + r;
#pragma unroll
            for (int c = 0; c < C2; ++c) {
                const int ch = min(lane * C2 + c, nchI - 1);
                qd[p][c] = ldg16(a.dnc + row * (a.I / 2) + ch * 16);
                if constexpr (FMT == FMT_NVFP4)
                    sd[p][c] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.dns) +
                                                                 row * (a.I / 16) + ch * 2);
                else
                    sd[p][c] = reinterpret_cast<const uint16_t*>(a.dns)[row * (a.I / 64) + (ch >> 1)];
            }
        }
    };

    const int n_up_pass = (u1 - u0 + 1) / 2;
    const int wu0 = share_lo(RU, blockIdx.x * kWaves, NW), wu1 = share_lo(RU, (blockIdx.x + 1) * kWaves, NW);
    const int wd0 = share_lo(RD, blockIdx.x * kDownWaves, NWD),
              wd1 = share_lo(RD, (blockIdx.x + 1) * kDownWaves, NWD);
    auto compute_up = [&](int p, int pass) {
        const int u = u0 + 2 * pass + seg;
        const bool ok = u < u1;
        const int slot = us0 + (u >= ubnd ? 1 : 0);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const bool chok = li * C + c < nchH;
            if constexpr (FMT == FMT_NVFP4) {
                const float s0 = chok ? e4m3fn_to_f32(su[p][c] & 0xffu) : 0.f;
                const float s1 = chok ? e4m3fn_to_f32(su[p][c] >> 8) : 0.f;
                acc += nvfp4_chunk_bf16(qu[p][c], xa[c], s0, s1);
            } else {
                const float sg = chok ? bf16_bits_to_f32(su[p][c]) : 0.f;
                acc = __builtin_fmaf(sg, int4_chunk_bf16(qu[p][c], xa[c]) - 136.0f * xs[c], acc);
            }
        }
        acc = seg_sum<32>(acc);
        const float g = __shfl(gu_l, slot, 64);
        if (li == 0 && ok) {
            const float rl = fmaxf(acc * g, 0.f);
            s_hrow[u - wu0] = rl * rl;
        }
    };
    // Per-tensor scales first, then the up loads, then the down loads
    // (independent of h), in that order, so each use waits only for what it
    // needs.
    compiler_fence();
    issue_up(0);
    compiler_fence();
    if (!ctl) issue_down(0);
    compiler_fence();

    // ---- U: compute h for this wave's rows
#pragma unroll
    for (int p = 0; p < kMaxUp; ++p)
        if (p < n_up_pass) compute_up(p, p);
    for (int pbase = kMaxUp; pbase < n_up_pass; pbase += kMaxUp) {  // only for small grids or large shapes
        issue_up(pbase);
#pragma unroll
        for (int p = 0; p < kMaxUp; ++p)
            if (pbase + p < n_up_pass) compute_up(p, pbase + p);
    }
    // ---- P: the control wave publishes the workgroup's h rows, then waits
    // for and stages the h of the slots the workgroup's down rows use
    __syncthreads();
    Q4MOE_PHASE(4);
    const int sl0 = wd1 > wd0 ? wd0 / a.H : 0, sl1 = wd1 > wd0 ? (wd1 - 1) / a.H : -1;  // at most two slots
    if (ctl) {
        for (int j = lane; j < wu1 - wu0; j += 64) {
            const int u = wu0 + j;
            const int slot = u / a.I, r = u - slot * a.I;
            const float v = s_hrow[j];
#pragma unroll
            for (int rp = 0; rp < kReplicas; ++rp) put_coherent(a.h + ((size_t)rp * a.K + slot) * a.I + r, v);
        }
        stores_done();  // only stores are in flight in this wave
        if (lane < kReplicas && wu1 > wu0) {  // lane t bumps copy t of the counters
            for (int s2 = wu0 / a.I; s2 <= (wu1 - 1) / a.I; ++s2) {
                const int n = min(wu1, (s2 + 1) * a.I) - max(wu0, s2 * a.I);
                atomicAdd(a.ctrl + FW_UP + s2 * kReplicas + lane, (uint32_t)n);
            }
        }
        if (lane == 0) {
            for (int s2 = sl0; s2 <= sl1; ++s2)
                spin_until(a.ctrl + FW_UP + s2 * kReplicas + rep, (uint32_t)a.I, flags);
        }
        compiler_fence();
        for (int s2 = sl0; s2 <= sl1; ++s2) {
            const float* src = a.h + ((size_t)rep * a.K + s2) * a.I;
            for (int j = lane; j < a.I / 2; j += 64) {
                const unsigned long long v = get_coherent2(src + 2 * j);
                s_h[s2 - sl0][2 * j] = __uint_as_float((uint32_t)v);
                s_h[s2 - sl0][2 * j + 1] = __uint_as_float((uint32_t)(v >> 32));
            }
        }
    }
    __syncthreads();
    Q4MOE_PHASE(5);

    float hv[C2][32];
    float hs[C2];
    int h_slot = -1;
    const int n_down = d1 - d0;
    auto compute_down = [&](int p, int idx) {
        const int d = d0 + idx;
        const int slot = ds0 + (d >= dbnd ? 1 : 0), r = d - slot * a.H;
        if (slot != h_slot) {  // wave-uniform
#pragma unroll
            for (int c = 0; c < C2; ++c) {
                const int ch = lane * C2 + c;
                hs[c] = 0.f;
                if (ch < nchI) {
                    const float4* hp = reinterpret_cast<const float4*>(&s_h[slot - sl0][ch * 32]);
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
            h_slot = slot;
        }
        float zz = 0.f;
#pragma unroll
        for (int c = 0; c < C2; ++c) {
            const bool chok = lane * C2 + c < nchI;
            if constexpr (FMT == FMT_NVFP4) {
                const float s0 = chok ? e4m3fn_to_f32(sd[p][c] & 0xffu) : 0.f;
                const float s1 = chok ? e4m3fn_to_f32(sd[p][c] >> 8) : 0.f;
                zz += nvfp4_chunk_f32(qd[p][c], hv[c], s0, s1);
            } else {
                const float sg = chok ? bf16_bits_to_f32(sd[p][c]) : 0.f;
                zz = __builtin_fmaf(sg, int4_chunk_f32(qd[p][c], hv[c]) - 8.0f * hs[c], zz);
            }
        }
        zz = seg_sum<64>(zz);
        const float g = __shfl(gd_l, slot, 64);
        if (lane == 0) put_coherent(a.z + (size_t)slot * a.H + r, (wsel[slot] * g) * zz);
    };
#pragma unroll
    for (int p = 0; p < kMaxDown; ++p)
        if (p < n_down) compute_down(p, p);
    for (int dbase = kMaxDown; dbase < n_down; dbase += kMaxDown) {  // only for small grids or large shapes
        issue_down(dbase);
#pragma unroll
        for (int p = 0; p < kMaxDown; ++p)
            if (dbase + p < n_down) compute_down(p, dbase + p);
    }

    // ---- C: publish the workgroup's down units per 64-row block; the
    // workgroup that completes a block sums it over the slots
    stores_done();
    __syncthreads();
    Q4MOE_PHASE(6);
    if (threadIdx.x == 0) {
        int nb = 0;
        int d = wd0;
        while (d < wd1) {  // runs of units inside one (slot, block)
            const int slot = d / a.H, r = d - slot * a.H;
            const int b = r / kRowBlock;
            const int end = min(wd1, slot * a.H + min(a.H, (b + 1) * kRowBlock));
            const uint32_t n = (uint32_t)(end - d);
            const uint32_t target = (uint32_t)a.K * (uint32_t)(min(a.H, (b + 1) * kRowBlock) - b * kRowBlock);
            const uint32_t old = atomicAdd(a.ctrl + FW_BLOCK + b, n);
            if (old + n == target && nb < kWaves) s_blocks[nb++] = b;
            d = end;
        }
        s_blocks[kWaves] = nb;
    }
    compiler_fence();
    __syncthreads();
    if (wave < s_blocks[kWaves]) {
        const int b = s_blocks[wave];
        const int r = b * kRowBlock + lane;
        if (r < a.H) {
            float yv = 0.f;
            for (int s2 = 0; s2 < a.K; ++s2) yv += get_coherent(a.z + (size_t)s2 * a.H + r);
            a.y32[r] = yv;
            a.y[r] = (uint16_t)f32_to_bf16_rne(yv);
        }
    }

    Q4MOE_PHASE(7);
    // ---- exit: the last workgroup out clears the counters for the next call
    if (threadIdx.x == 0) {
        const uint32_t done = atomicAdd(a.ctrl + FW_EXIT, 1u);
        if (done == gridDim.x - 1) {
            for (int i = 0; i < kReplicas; ++i) atomicExch(a.ctrl + FW_ROUTER + i, 0u);
            for (int i = 0; i < 8 * kReplicas; ++i) atomicExch(a.ctrl + FW_UP + i, 0u);
            for (int b = 0; b < kFusedMaxBlocks; ++b) atomicExch(a.ctrl + FW_BLOCK + b, 0u);
            atomicExch(a.ctrl + FW_EXIT, 0u);
        }
    }
}

}  // namespace q4moe
