// libq4moe C-ABI: host-side validation, workspace layout and launches.
// Declarations, argument meaning, layouts and error behaviour: include/q4moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "q4moe.h"
#include "q4moe_fused.hpp"
#include "q4moe_w4a4.hpp"
#include "q4moe_grouped16.hpp"
#include "q4moe_fp8gemv.hpp"
#include "q4moe_wquant.hpp"
#include "q4moe_shared.hpp"

using namespace q4moe;

namespace {

thread_local char g_err[512] = "";

q4moe_status fail(q4moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
constexpr size_t up_to(size_t n, size_t a = kAlign) { return (n + a - 1) / a * a; }

constexpr int kMaxDim = 4096;

q4moe_status device_ready() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(Q4MOE_EDEVICE, "no HIP device: %s", hipGetErrorString(e));
    return Q4MOE_OK;
}

q4moe_status launched(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(Q4MOE_EDEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return Q4MOE_OK;
}

q4moe_status check_router(const q4moe_router* r) {
    if (!r) return fail(Q4MOE_EINVAL, "router descriptor is NULL");
    if (!r->w_g || !r->bias) return fail(Q4MOE_EINVAL, "router w_g / bias is NULL");
    if (r->n_experts < 1 || r->n_experts > 256)
        return fail(Q4MOE_EINVAL, "router n_experts %d outside [1, 256]", r->n_experts);
    if (r->hidden < 32 || r->hidden % 32 != 0 || r->hidden > kMaxDim)
        return fail(Q4MOE_EINVAL, "router hidden %d must be a multiple of 32 in [32, %d]", r->hidden, kMaxDim);
    if (r->top_k < 1 || r->top_k > 8 || r->top_k > r->n_experts)
        return fail(Q4MOE_EINVAL, "top_k %d outside [1, min(8, n_experts)]", r->top_k);
    if (!aligned(r->w_g, 16)) return fail(Q4MOE_EALIGN, "router w_g not 16-byte aligned");
    if (!aligned(r->bias, 4)) return fail(Q4MOE_EALIGN, "router bias not 4-byte aligned");
    return Q4MOE_OK;
}

q4moe_status check_experts(const q4moe_experts* ex, const q4moe_router* r) {
    if (!ex) return fail(Q4MOE_EINVAL, "experts descriptor is NULL");
    if (ex->fmt != Q4MOE_NVFP4 && ex->fmt != Q4MOE_INT4_G64)
        return fail(Q4MOE_EINVAL, "unknown expert format %d", ex->fmt);
    if (ex->n_experts != r->n_experts || ex->hidden != r->hidden)
        return fail(Q4MOE_EINVAL, "experts (%d x hidden %d) do not match the router (%d x hidden %d)",
                    ex->n_experts, ex->hidden, r->n_experts, r->hidden);
    const int q = ex->fmt == Q4MOE_NVFP4 ? 32 : 64;
    if (ex->hidden % q != 0 || ex->inter < q || ex->inter % q != 0 || ex->inter > kMaxDim)
        return fail(Q4MOE_EINVAL, "hidden %d / inter %d must be multiples of %d in [%d, %d]", ex->hidden,
                    ex->inter, q, q, kMaxDim);
    if (!ex->up_codes || !ex->up_scales || !ex->down_codes || !ex->down_scales)
        return fail(Q4MOE_EINVAL, "expert code / scale pointer is NULL");
    if (ex->fmt == Q4MOE_NVFP4 && (!ex->up_gscale || !ex->down_gscale))
        return fail(Q4MOE_EINVAL, "NVFP4 experts need up_gscale and down_gscale");
    if (ex->fmt == Q4MOE_INT4_G64 && (ex->up_gscale || ex->down_gscale))
        return fail(Q4MOE_EINVAL, "INT4_G64 experts take no per-tensor scale (pass NULL)");
    if (!aligned(ex->up_codes, 16) || !aligned(ex->down_codes, 16))
        return fail(Q4MOE_EALIGN, "expert codes not 16-byte aligned");
    if (!aligned(ex->up_scales, 4) || !aligned(ex->down_scales, 4))
        return fail(Q4MOE_EALIGN, "expert scales not 4-byte aligned");
    if ((ex->up_gscale && !aligned(ex->up_gscale, 4)) || (ex->down_gscale && !aligned(ex->down_gscale, 4)))
        return fail(Q4MOE_EALIGN, "expert gscale not 4-byte aligned");
    return Q4MOE_OK;
}

// ---------------------------------------------------------------------------
// Workspace layouts
// ---------------------------------------------------------------------------

// Every workspace starts with the same prefix at the same offsets, whatever
// the entry point, shape or token count: the control words, then the tag
// area of the one-launch decode, sized for the largest supported shapes.
// Only the one-launch decode writes the tag area, and it accepts a tag only
// when it carries the current call's epoch (one more than the last completed
// call's), so values of earlier calls never match and no other entry point
// can leave a value there that a later one-launch call would take.  Each
// entry point's own scratch follows the prefix.
constexpr int kMaxExperts = 256, kMaxTopK = 8;
constexpr size_t kScTagOff = up_to(CTRL_WORDS * 4);
constexpr size_t kHTagOff = kScTagOff + up_to((size_t)kReplicas * kMaxExperts * 8);
constexpr size_t kZTagOff = kHTagOff + up_to((size_t)kReplicas * kMaxTopK * kMaxDim * 8);
constexpr size_t kHqTagOff = kZTagOff + up_to((size_t)(kMaxTopK + 1) * kMaxDim * 8);
constexpr size_t kYTagOff = kHqTagOff + up_to((size_t)kReplicas * (kMaxDim / 4) * 8);
constexpr size_t kDoneTagOff = kYTagOff + up_to((size_t)kReplicas * (kMaxDim / 2) * 8);
constexpr size_t kPrefixBytes = kDoneTagOff + up_to((size_t)kReplicas * 64 * 8);

struct RouterWs {
    size_t ctrl, logits, ids, w, total;
};

RouterWs router_ws(int E, int K, int T) {
    RouterWs l;
    size_t o = kPrefixBytes;
    l.ctrl = 0;
    l.logits = o;
    o += up_to((size_t)T * E * 4);
    l.ids = o;
    o += up_to((size_t)T * K * 4);
    l.w = o;
    o += up_to((size_t)T * K * 4);
    l.total = o;
    return l;
}

struct DecodeWs {
    RouterWs r;
    size_t sc_tag, h_tag, z_tag, y_tag, done_tag, h, y32, zw, hq_tag, sh_xq, sh_h, sh_hq, sh_z, xq_c, xq_s, hq_c, hq_s;
    // the grouped path (more than kSmallT tokens): dispatch, fp16 staging
    size_t counts, offsets, lists, perm, inv, act, n_act, x16, xexp, h16, hexp;
    // the shared expert through the grouped GEMMs (one-expert dispatch)
    size_t sh_act, sh_nact, sh_perm, sh_gate, sh_x16, sh_xexp, sh_h16, sh_hexp;
    size_t total;
};

// Whether the W4A16 decode of T tokens takes the grouped path (measured
// cold crossovers at the full shapes, 128 x 2688 x 1856 top-6): NVFP4 above
// 4 tokens (at 5 tokens the grouped path takes 93 us, the 8-token
// small-batch kernels 106 us), int4 above 2 (its small-batch kernels stream
// each expert once per token and slot: 100 us against 87 us at 3 tokens).
bool w4a16_grouped(int fmt, int T) { return fmt == Q4MOE_NVFP4 ? T > kSmallT : T > 2; }

// S: the shared expert's intermediate size (0: no shared expert); a4: the
// W4A4 decode (NVFP4 activation code taps); grouped: the grouped path's
// buffers (they follow every other buffer, so the tap offsets do not depend
// on it).
DecodeWs decode_ws(int E, int H, int I, int K, int T, int S = 0, bool a4 = false, bool grouped = false,
                   bool sh_grouped = false) {
    DecodeWs l;
    l.r = router_ws(E, K, T);
    // the one-launch decode's tags, in the common prefix:
    l.sc_tag = kScTagOff;  // (score, epoch) pairs [kReplicas][E]
    l.h_tag = kHTagOff;    // (h, epoch) pairs [kReplicas][K][I] (W4A4: codes and scales)
    l.z_tag = kZTagOff;    // (w * g * z, epoch) pairs [K + 1][H]; slot K: the shared expert
    l.hq_tag = kHqTagOff;  // shared expert: (four h codes, epoch) [kReplicas][S / 4]
    l.y_tag = kYTagOff;    // a chained stack's y for its next layer: (two bf16, epoch) [kReplicas][H / 2]
    l.done_tag = kDoneTagOff;  // a stack's combined blocks of y: (0, epoch) [kReplicas][64]
    size_t o = l.r.total;
    l.sh_xq = o;   // shared expert taps [T][H], [T][S], [T][S], and its z [T][H]
    o += up_to(S > 0 ? (size_t)T * H : 0);
    l.sh_h = o;
    o += up_to((size_t)T * S * 4);
    l.sh_hq = o;
    o += up_to((size_t)T * S);
    l.sh_z = o;
    o += up_to(S > 0 ? (size_t)T * H * 4 : 0);
    l.xq_c = o;    // W4A4 taps: x codes and scales, h codes and scales
    o += up_to(a4 ? (size_t)T * H / 2 : 0);
    l.xq_s = o;
    o += up_to(a4 ? (size_t)T * H / 16 : 0);
    l.hq_c = o;
    o += up_to(a4 ? (size_t)T * K * I / 2 : 0);
    l.hq_s = o;
    o += up_to(a4 ? (size_t)T * K * I / 16 : 0);
    l.h = o;       // h tap
    o += up_to((size_t)T * K * I * 4);
    l.y32 = o;
    o += up_to((size_t)T * H * 4);
    l.zw = o;      // multi-token path: w * g * z per (token, slot) pair
    o += up_to((size_t)T * K * H * 4);
    // the grouped path's own buffers
    const size_t rows = grouped ? (size_t)T * K : 0;
    auto take = [&](size_t& off, size_t bytes) {
        off = o;
        o += up_to(bytes);
    };
    take(l.counts, grouped ? (size_t)E * 4 : 0);
    take(l.offsets, grouped ? (size_t)(E + 1) * 4 : 0);
    take(l.lists, grouped ? (size_t)E * T * 4 : 0);
    take(l.perm, rows * 4);
    take(l.inv, rows * 4);
    take(l.act, grouped ? (size_t)E * 16 : 0);
    take(l.n_act, grouped ? 4 : 0);
    take(l.x16, grouped ? (size_t)T * H * 2 : 0);
    take(l.xexp, grouped ? (size_t)T * 4 : 0);
    take(l.h16, rows * 2 * I * 2);
    take(l.hexp, rows * 4);
    // the shared expert's grouped buffers (after every other buffer)
    const size_t st = sh_grouped ? (size_t)T : 0;
    take(l.sh_act, sh_grouped ? 16 : 0);
    take(l.sh_nact, sh_grouped ? 4 : 0);
    take(l.sh_perm, st * 4);
    take(l.sh_gate, st * 4);
    take(l.sh_x16, st * H * 2);
    take(l.sh_xexp, st * 4);
    take(l.sh_h16, st * 2 * S * 2);
    take(l.sh_hexp, st * 4);
    l.total = o;
    return l;
}

// Workgroups of a persistent kernel: as many as fit on the device at once,
// at most `want`; 0 if the occupancy query fails.
template <typename K>
int persistent_grid(K kernel, int block, int want) {
    int dev = 0, per_cu = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu < 1)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
    return std::max(1, std::min(want, per_cu * cus));
}

// Workgroups of the fused decode that fit on the device at once (so that
// every workgroup is resident and every wait can be satisfied), cached per
// device and kernel variant.
constexpr int kMaxDevices = 64;
constexpr int kFusedVariants = 32;  // 8 shapes x (plain, shared, W4A4)
int g_fused_grid[kMaxDevices][kFusedVariants];

template <int FMT, int C, int C2, bool SH, bool A4>
int fused_grid(int dev, int variant) {
    if (dev < 0 || dev >= kMaxDevices) return 0;
    int& cached = g_fused_grid[dev][variant];
    if (cached != 0) return cached;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_fused<FMT, C, C2, SH, A4>, 64 * kWaves, 0) !=
        hipSuccess)
        return 0;
    cached = cus * (per_cu < 1 ? 0 : 1);
    return cached;
}

// Whether a one-launch decode of this shape runs on `grid` workgroups.  The
// router needs one workgroup per expert; every wave's up rows must fit in
// kMaxUp passes (all loads in flight at once), a workgroup stages at most
// kMaxWgUp up rows, every down unit (kDownRows rows of one slot) needs a
// wave, and a workgroup's kWaves units span at most two slots.  Otherwise
// the caller uses separate launches.
bool fused_fits(const FusedArgs& a, int grid, bool SH, bool A4) {
    const long long RU = (long long)a.K * a.I;
    const long long nw = (long long)grid * kWaves;
    const long long dpu = (a.H + kDownRows - 1) / kDownRows;
    if (grid < a.E || grid > CTRL_WORDS - FW_EPOCH || (RU + nw - 1) / nw > 2 * kMaxUp ||
        (RU + grid - 1) / grid > kMaxWgUp || a.K * dpu > nw || dpu < kWaves - 1)
        return false;
    // block scales are read as 8-byte pieces of a row's region (at least 8
    // bytes: hidden >= 256) and 16-byte pieces of a down unit's whole rows
    if (a.H < 256 || a.H % kDownRows != 0) return false;
    // shared expert: at most 4 h-code quads (16 up rows) per workgroup and
    // two down rows per wave
    if (SH && (a.S / 4 > 4LL * grid || a.H > 2 * nw)) return false;
    // W4A4: a workgroup's up rows are whole 16-row blocks
    if (A4) {
        const long long wg_rows = 16 * ((RU / 16 + grid - 1) / grid);
        if (RU % 16 != 0 || wg_rows > kMaxWgUp || (wg_rows + kWaves - 1) / kWaves > 2 * kMaxUp) return false;
    }
    return true;
}

template <int FMT, int C, int C2, bool SH, bool A4>
q4moe_status launch_fused_v(const FusedArgs& a, hipStream_t s, int variant) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(Q4MOE_EDEVICE, "hipGetDevice failed");
    const int grid = fused_grid<FMT, C, C2, SH, A4>(dev, variant);
    if (!fused_fits(a, grid, SH, A4)) return Q4MOE_EUNSUPPORTED;
    hipLaunchKernelGGL((k_decode_fused<FMT, C, C2, SH, A4>), dim3(grid), dim3(64 * kWaves), 0, s, a);
    return launched("fused decode");
}

// The stacked decode: the same grid rule (one workgroup per CU, all resident).
int g_stack_grid[kMaxDevices][16];

template <int FMT, int C, int C2>
q4moe_status launch_stack_v(const StackArgs& sa, hipStream_t s, int variant) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(Q4MOE_EDEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return Q4MOE_EUNSUPPORTED;
    int& grid = g_stack_grid[dev][variant];
    if (grid == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_stack<FMT, C, C2>, 64 * kWaves, 0) !=
                hipSuccess)
            return Q4MOE_EUNSUPPORTED;
        grid = per_cu < 1 ? -1 : cus;
    }
    if (grid < 0 || !fused_fits(sa.a, grid, false, false)) return Q4MOE_EUNSUPPORTED;
    hipLaunchKernelGGL((k_decode_stack<FMT, C, C2>), dim3(grid), dim3(64 * kWaves), 0, s, sa);
    return launched("stacked decode");
}

template <int FMT>
q4moe_status launch_stack(const StackArgs& sa, hipStream_t s) {
    const int C = (sa.a.H / 32 + 31) / 32, C2 = (sa.a.I / 32 + 63) / 64;
    const int v = (C - 1) * 2 + (C2 - 1);
    const int slot = v + (FMT == FMT_NVFP4 ? 0 : 8);
    switch (v) {
        case 0: return launch_stack_v<FMT, 1, 1>(sa, s, slot);
        case 1: return launch_stack_v<FMT, 1, 2>(sa, s, slot);
        case 2: return launch_stack_v<FMT, 2, 1>(sa, s, slot);
        case 3: return launch_stack_v<FMT, 2, 2>(sa, s, slot);
        case 4: return launch_stack_v<FMT, 3, 1>(sa, s, slot);
        case 5: return launch_stack_v<FMT, 3, 2>(sa, s, slot);
        case 6: return launch_stack_v<FMT, 4, 1>(sa, s, slot);
        case 7: return launch_stack_v<FMT, 4, 2>(sa, s, slot);
    }
    return Q4MOE_EUNSUPPORTED;
}

template <int FMT, bool SH = false, bool A4 = false>
q4moe_status launch_fused(const FusedArgs& a, hipStream_t s) {
    const int C = (a.H / 32 + 31) / 32, C2 = (a.I / 32 + 63) / 64;
    const int v = (C - 1) * 2 + (C2 - 1);
    const int slot = v + (SH ? 8 : 0) + (A4 ? 16 : 0);  // grid cache entry
    switch (v) {
        case 0: return launch_fused_v<FMT, 1, 1, SH, A4>(a, s, slot);
        case 1: return launch_fused_v<FMT, 1, 2, SH, A4>(a, s, slot);
        case 2: return launch_fused_v<FMT, 2, 1, SH, A4>(a, s, slot);
        case 3: return launch_fused_v<FMT, 2, 2, SH, A4>(a, s, slot);
        case 4: return launch_fused_v<FMT, 3, 1, SH, A4>(a, s, slot);
        case 5: return launch_fused_v<FMT, 3, 2, SH, A4>(a, s, slot);
        case 6: return launch_fused_v<FMT, 4, 1, SH, A4>(a, s, slot);
        case 7: return launch_fused_v<FMT, 4, 2, SH, A4>(a, s, slot);
    }
    return Q4MOE_EUNSUPPORTED;
}

struct W4a4Ws {
    RouterWs r;
    size_t counts, offsets, lists, perm, inv, xq_codes, xq_scales, h32, hq_codes, hq_scales, z, y32, total;
};

W4a4Ws w4a4_ws(int E, int H, int I, int K, int T) {
    W4a4Ws l;
    l.r = router_ws(E, K, T);
    const size_t rows = (size_t)T * K;
    size_t o = l.r.total;
    auto take = [&](size_t& off, size_t bytes) {
        off = o;
        o += up_to(bytes);
    };
    take(l.counts, (size_t)E * 4);
    take(l.offsets, (size_t)(E + 1) * 4);
    take(l.lists, (size_t)E * T * 4);
    take(l.perm, rows * 4);
    take(l.inv, rows * 4);
    take(l.xq_codes, (size_t)T * H / 2);
    take(l.xq_scales, (size_t)T * H / 16);
    take(l.h32, rows * I * 4);
    take(l.hq_codes, rows * I / 2);
    take(l.hq_scales, rows * I / 16);
    take(l.z, rows * H * 4);
    take(l.y32, (size_t)T * H * 4);
    l.total = o;
    return l;
}

q4moe_status check_w4a4(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    q4moe_status st = check_router(r);
    if (st != Q4MOE_OK) return st;
    if ((st = check_experts(ex, r)) != Q4MOE_OK) return st;
    if (ex->fmt != Q4MOE_NVFP4) return fail(Q4MOE_EUNSUPPORTED, "the W4A4 path takes NVFP4 experts only");
    if (ex->hidden % 64 != 0 || ex->inter % 64 != 0)
        return fail(Q4MOE_EUNSUPPORTED, "W4A4 needs hidden and inter multiples of 64 (got %d, %d)", ex->hidden,
                    ex->inter);
    if (n_tok < 1 || n_tok > 65536) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 65536]", n_tok);
    return Q4MOE_OK;
}

// Workgroups of the lm_head GEMV at most (its persistent grid is capped here).
constexpr int kMaxGemvBlocks = 4096;

struct GemvWs {
    size_t ctrl, keys, total;
};

GemvWs gemv_ws(int T) {
    GemvWs l;
    l.ctrl = 0;
    l.keys = kPrefixBytes;
    l.total = l.keys + up_to((size_t)kMaxGemvBlocks * T * 8);
    return l;
}

// The FP8 GEMV: the keys, then its activation code tap [T][cols].
struct Fp8GemvWs {
    size_t keys, xq, total;
};

Fp8GemvWs fp8_gemv_ws(int T, int cols) {
    Fp8GemvWs l;
    l.keys = kPrefixBytes;
    l.xq = l.keys + up_to((size_t)kMaxGemvBlocks * T * 8);
    l.total = l.xq + up_to((size_t)T * cols);
    return l;
}

q4moe_status check_ws(const void* ws, size_t have, size_t need) {
    if (!ws) return fail(Q4MOE_EINVAL, "workspace is NULL");
    if (!aligned(ws, 16)) return fail(Q4MOE_EALIGN, "workspace not 16-byte aligned");
    if (have < need) return fail(Q4MOE_EWORKSPACE, "workspace %zu bytes, need %zu", have, need);
    return Q4MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

RouterArgs router_args(const q4moe_router* r, const uint16_t* x, int T, void* ws, const RouterWs& l,
                       int32_t* ids_out, float* w_out, float* logits_out) {
    RouterArgs a;
    a.wg = r->w_g;
    a.bias = r->bias;
    a.x = x;
    a.E = r->n_experts;
    a.H = r->hidden;
    a.T = T;
    a.K = r->top_k;
    a.logits = at<float>(ws, l.logits);
    a.ids = at<int32_t>(ws, l.ids);
    a.w = at<float>(ws, l.w);
    a.ids_out = ids_out;
    a.w_out = w_out;
    a.logits_out = logits_out;
    return a;
}

// The MFMA router GEMM: two token blocks per workgroup (the router matrix
// read half as often) when that still leaves 256 workgroups, else one.  The
// logits are the same either way.
void launch_router_gemm(const RouterArgs& a, hipStream_t s) {
    const unsigned ge = (unsigned)((a.E + kRouterTile - 1) / kRouterTile);
    const unsigned gt2 = (unsigned)((a.T + 2 * kRouterTile - 1) / (2 * kRouterTile));
    if (gt2 * ge >= 256)
        hipLaunchKernelGGL(k_router_gemm<2>, dim3(gt2, ge), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL(k_router_gemm<1>, dim3((unsigned)((a.T + kRouterTile - 1) / kRouterTile), ge), dim3(512),
                           0, s, a);
}

q4moe_status launch_router(const RouterArgs& a, hipStream_t s) {
    if (a.T >= 16) {  // many tokens: the MFMA router GEMM
        launch_router_gemm(a, s);
    } else {
        dim3 g1(a.E, (a.T + 3) / 4);
        hipLaunchKernelGGL(k_router_logits, g1, dim3(256), 0, s, a);
    }
    q4moe_status st = launched("router logits");
    if (st != Q4MOE_OK) return st;
    hipLaunchKernelGGL(k_topk, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
    return launched("router top-k");
}

template <int FMT>
q4moe_status launch_up(const MoeArgs& a, hipStream_t s) {
    dim3 grid((a.I + 7) / 8, a.T * a.K);
    const int C = (a.H / 32 + 31) / 32;
    switch (C) {
        case 1: hipLaunchKernelGGL((k_up<1, FMT>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_up<2, FMT>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((k_up<3, FMT>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_up<4, FMT>), grid, dim3(256), 0, s, a); break;
        default: return fail(Q4MOE_EUNSUPPORTED, "hidden %d too wide", a.H);
    }
    return launched("up projection");
}

template <int FMT, int T>
q4moe_status launch_down_t(const MoeArgs& a, hipStream_t s) {
    dim3 grid((a.H + 15) / 16);
    const int C = (a.I / 32 + 63) / 64;
    switch (C) {
        case 1: hipLaunchKernelGGL((k_down<1, FMT, T>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_down<2, FMT, T>), grid, dim3(256), 0, s, a); break;
        default: return fail(Q4MOE_EUNSUPPORTED, "inter %d too wide", a.I);
    }
    return launched("down projection");
}

template <int FMT>
q4moe_status launch_down(const MoeArgs& a, hipStream_t s) {
    switch (a.T) {
        case 1: return launch_down_t<FMT, 1>(a, s);
        case 2: return launch_down_t<FMT, 2>(a, s);
        case 3: return launch_down_t<FMT, 3>(a, s);
        default: return launch_down_t<FMT, 4>(a, s);
    }
}

// NJ instance of the small-batch kernels for a reduction of `cols` (128
// columns per piece; pieces past cols are masked).
inline int small_nj(int cols) {
    const int nj = (cols + 127) / 128;
    return nj <= 8 ? 8 : nj <= 15 ? 15 : nj <= 16 ? 16 : nj <= 21 ? 21 : nj <= 24 ? 24 : 32;
}

template <int TM, bool A4>
q4moe_status launch_small_t(const SmallMoeArgs& a, hipStream_t s) {
    const int pairs = a.T * a.K;
    const dim3 gu((a.I + 63) / 64, pairs), gd((a.H + 63) / 64, pairs);
#define Q4_SMALL(KERN, NJ, G) hipLaunchKernelGGL((KERN<NJ, TM, A4>), G, dim3(256), 0, s, a)
#define Q4_SMALL_NJ(KERN, NJV, G)              \
    switch (NJV) {                             \
        case 8: Q4_SMALL(KERN, 8, G); break;   \
        case 15: Q4_SMALL(KERN, 15, G); break; \
        case 16: Q4_SMALL(KERN, 16, G); break; \
        case 21: Q4_SMALL(KERN, 21, G); break; \
        case 24: Q4_SMALL(KERN, 24, G); break; \
        default: Q4_SMALL(KERN, 32, G); break; \
    }
    Q4_SMALL_NJ(k_small_up, small_nj(a.H), gu);
    q4moe_status st = launched("small-batch up projection");
    if (st != Q4MOE_OK) return st;
    Q4_SMALL_NJ(k_small_down, small_nj(a.I), gd);
    if ((st = launched("small-batch down projection")) != Q4MOE_OK) return st;
#undef Q4_SMALL_NJ
#undef Q4_SMALL
    hipLaunchKernelGGL(k_small_combine, dim3((a.T * a.H + 255) / 256), dim3(256), 0, s, a);
    return launched("small-batch combine");
}

// The small-batch kernels: up to 4 tokens the 4-token instances; the W4A4
// form also takes 5..8 tokens with the 8-token instances (the W4A16 decode
// sends more than 4 tokens to the grouped path).
q4moe_status launch_small(const SmallMoeArgs& a, bool a4, hipStream_t s) {
    if (a.T <= kSmallT) return a4 ? launch_small_t<kSmallT, true>(a, s) : launch_small_t<kSmallT, false>(a, s);
    if (!a4) return fail(Q4MOE_EUNSUPPORTED, "the W4A16 small-batch kernels take up to %d tokens", kSmallT);
    return launch_small_t<kSmallT8, true>(a, s);
}

// The grouped W4A16 path for more than kSmallT tokens (hidden and inter
// multiples of 64): router, dispatch, fp16 staging, two grouped MFMA GEMMs
// and the combine, in order on one stream.
q4moe_status launch_grouped16(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x, int T, uint16_t* y,
                              int32_t* ids_out, float* w_out, void* ws, const DecodeWs& l, hipStream_t s,
                              const float* zsh = nullptr) {
    const int E = r->n_experts, H = ex->hidden, I = ex->inter, K = r->top_k;
    RouterArgs ra = router_args(r, x, T, ws, l.r, ids_out, w_out, nullptr);
    q4moe_status st = launch_router(ra, s);
    if (st != Q4MOE_OK) return st;

    DispatchArgs da;
    da.ids = ra.ids;
    da.T = T;
    da.K = K;
    da.E = E;
    da.counts = at<int32_t>(ws, l.counts);
    da.lists = at<int32_t>(ws, l.lists);
    da.offsets = at<int32_t>(ws, l.offsets);
    da.perm = at<int32_t>(ws, l.perm);
    da.inv = at<int32_t>(ws, l.inv);
    da.act = at<int4>(ws, l.act);
    da.n_act = at<int32_t>(ws, l.n_act);
    hipLaunchKernelGGL(k_dispatch, dim3(E), dim3(64), 0, s, da);
    if ((st = launched("dispatch")) != Q4MOE_OK) return st;
    hipLaunchKernelGGL(k_dispatch_scan, dim3(E), dim3(256), 0, s, da);
    if ((st = launched("dispatch scan")) != Q4MOE_OK) return st;

    StageArgs sx;
    sx.cols = H;
    sx.xb = x;
    sx.hf = nullptr;
    sx.out = at<_Float16>(ws, l.x16);
    sx.exps = at<int32_t>(ws, l.xexp);
    hipLaunchKernelGGL(k_stage_x16, dim3(T), dim3(256), 0, s, sx);
    if ((st = launched("x staging")) != Q4MOE_OK) return st;

    const bool nv = ex->fmt == Q4MOE_NVFP4;
    GemmA16Args gu;
    gu.N = I;
    gu.Kd = H;
    gu.K = K;
    gu.wc = ex->up_codes;
    gu.wsc = static_cast<const uint8_t*>(ex->up_scales);
    gu.wg = ex->up_gscale;
    gu.a16 = sx.out;
    gu.aexp = sx.exps;
    gu.act = da.act;
    gu.n_act = da.n_act;
    gu.perm = da.perm;
    gu.gate = ra.w;
    gu.out = at<float>(ws, l.h);
    const dim3 grid_up((I + kGemmBN - 1) / kGemmBN, E);
    const size_t lds_up = (size_t)kGemmBN * (nv ? H / 16 : H / 32) + 16;
    if (nv)
        hipLaunchKernelGGL((k_grouped_a16<EPI_UP, FMT_NVFP4>), grid_up, dim3(256), lds_up, s, gu);
    else
        hipLaunchKernelGGL((k_grouped_a16<EPI_UP, FMT_INT4>), grid_up, dim3(256), lds_up, s, gu);
    if ((st = launched("grouped up gemm")) != Q4MOE_OK) return st;

    StageArgs sh;
    sh.cols = I;
    sh.xb = nullptr;
    sh.hf = gu.out;
    sh.out = at<_Float16>(ws, l.h16);
    sh.exps = at<int32_t>(ws, l.hexp);
    hipLaunchKernelGGL(k_stage_h16, dim3(T * K), dim3(256), 0, s, sh);
    if ((st = launched("h staging")) != Q4MOE_OK) return st;

    GemmA16Args gd = gu;
    gd.N = H;
    gd.Kd = I;
    gd.wc = ex->down_codes;
    gd.wsc = static_cast<const uint8_t*>(ex->down_scales);
    gd.wg = ex->down_gscale;
    gd.a16 = sh.out;
    gd.aexp = sh.exps;
    gd.out = at<float>(ws, l.zw);
    const dim3 grid_dn((H + kGemmBN - 1) / kGemmBN, E);
    const size_t lds_dn = (size_t)kGemmBN * (nv ? I / 16 : I / 32) + 16;
    if (nv)
        hipLaunchKernelGGL((k_grouped_a16<EPI_DOWN, FMT_NVFP4>), grid_dn, dim3(256), lds_dn, s, gd);
    else
        hipLaunchKernelGGL((k_grouped_a16<EPI_DOWN, FMT_INT4>), grid_dn, dim3(256), lds_dn, s, gd);
    if ((st = launched("grouped down gemm")) != Q4MOE_OK) return st;

    SmallMoeArgs b;
    b.T = T;
    b.H = H;
    b.K = K;
    b.zw = gd.out;
    b.y32 = at<float>(ws, l.y32);
    b.y = y;
    b.zsh = zsh;
    hipLaunchKernelGGL(k_small_combine, dim3((T * H + 255) / 256), dim3(256), 0, s, b);
    return launched("combine");
}

// The shared expert as the grouped GEMMs see it: FP8 per-tensor W8A8, or a
// 4-bit W4A16 expert (NVFP4 or int4-g64).
struct SharedDense {
    int wf, S;
    const uint8_t *upc, *ups, *dnc, *dns;
    const float *upg, *dng;
    float up_gs, dn_gs, up_in, dn_in;  // FP8: weight scale * input scale, input scales
};

SharedDense shared_dense(const q4moe_shared_fp8* sh, const q4moe_experts* sh4) {
    SharedDense d;
    if (sh) {
        d.wf = FMT_FP8;
        d.S = sh->inter;
        d.upc = sh->up_codes;
        d.dnc = sh->down_codes;
        d.ups = d.dns = nullptr;
        d.upg = d.dng = nullptr;
        d.up_gs = sh->up_wscale * sh->up_iscale;
        d.dn_gs = sh->down_wscale * sh->down_iscale;
        d.up_in = sh->up_iscale;
        d.dn_in = sh->down_iscale;
    } else {
        d.wf = sh4->fmt == Q4MOE_NVFP4 ? FMT_NVFP4 : FMT_INT4;
        d.S = sh4->inter;
        d.upc = sh4->up_codes;
        d.dnc = sh4->down_codes;
        d.ups = static_cast<const uint8_t*>(sh4->up_scales);
        d.dns = static_cast<const uint8_t*>(sh4->down_scales);
        d.upg = sh4->up_gscale;
        d.dng = sh4->down_gscale;
        d.up_gs = d.dn_gs = d.up_in = d.dn_in = 1.0f;
    }
    return d;
}

// The shared expert for T tokens through the grouped GEMMs, as a one-expert
// dispatch (every token a row with gate 1): zsh [T][H] = its output, with
// the taps sh_xq / sh_hq (FP8 codes) and sh_h (relu(u)^2).  hidden a
// multiple of 64.
q4moe_status launch_shared_grouped(const SharedDense& d, const uint16_t* x, int T, int H, void* ws, const DecodeWs& l,
                                   hipStream_t s) {
    q4moe_status st;
    int4* act = at<int4>(ws, l.sh_act);
    int32_t* nact = at<int32_t>(ws, l.sh_nact);
    int32_t* perm = at<int32_t>(ws, l.sh_perm);
    float* gate = at<float>(ws, l.sh_gate);
    hipLaunchKernelGGL(k_dispatch_all, dim3((T + 255) / 256), dim3(256), 0, s, T, act, nact, perm, gate);
    if ((st = launched("shared expert dispatch")) != Q4MOE_OK) return st;
    const bool f8 = d.wf == FMT_FP8;
    StageArgs sx;
    sx.cols = H;
    sx.xb = x;
    sx.hf = nullptr;
    sx.out = at<_Float16>(ws, l.sh_x16);
    sx.exps = at<int32_t>(ws, l.sh_xexp);
    sx.iscale = d.up_in;
    sx.codes = f8 ? at<uint8_t>(ws, l.sh_xq) : nullptr;
    if (f8)
        hipLaunchKernelGGL((k_stage_fp8<true>), dim3(T), dim3(256), 0, s, sx);
    else
        hipLaunchKernelGGL(k_stage_x16, dim3(T), dim3(256), 0, s, sx);
    if ((st = launched("shared expert x staging")) != Q4MOE_OK) return st;
    GemmA16Args gu;
    gu.N = d.S;
    gu.Kd = H;
    gu.K = 1;
    gu.wc = d.upc;
    gu.wsc = d.ups;
    gu.wg = d.upg;
    gu.gs = d.up_gs;
    gu.a16 = sx.out;
    gu.aexp = sx.exps;
    gu.act = act;
    gu.n_act = nact;
    gu.perm = perm;
    gu.gate = gate;
    gu.out = at<float>(ws, l.sh_h);
    const dim3 grid_up((d.S + kGemmBN - 1) / kGemmBN, 1);
    const size_t lds_up = d.wf == FMT_NVFP4 ? (size_t)kGemmBN * (H / 16) + 16 : d.wf == FMT_INT4 ? (size_t)kGemmBN * (H / 32) + 16 : 16;
    if (d.wf == FMT_FP8)
        hipLaunchKernelGGL((k_grouped_a16<EPI_UP, FMT_FP8>), grid_up, dim3(256), lds_up, s, gu);
    else if (d.wf == FMT_NVFP4)
        hipLaunchKernelGGL((k_grouped_a16<EPI_UP, FMT_NVFP4>), grid_up, dim3(256), lds_up, s, gu);
    else
        hipLaunchKernelGGL((k_grouped_a16<EPI_UP, FMT_INT4>), grid_up, dim3(256), lds_up, s, gu);
    if ((st = launched("shared expert up gemm")) != Q4MOE_OK) return st;
    StageArgs sh;
    sh.cols = d.S;
    sh.xb = nullptr;
    sh.hf = gu.out;
    sh.out = at<_Float16>(ws, l.sh_h16);
    sh.exps = at<int32_t>(ws, l.sh_hexp);
    sh.iscale = d.dn_in;
    sh.codes = f8 ? at<uint8_t>(ws, l.sh_hq) : nullptr;
    if (f8)
        hipLaunchKernelGGL((k_stage_fp8<false>), dim3(T), dim3(256), 0, s, sh);
    else
        hipLaunchKernelGGL(k_stage_h16, dim3(T), dim3(256), 0, s, sh);
    if ((st = launched("shared expert h staging")) != Q4MOE_OK) return st;
    GemmA16Args gd = gu;
    gd.N = H;
    gd.Kd = d.S;
    gd.wc = d.dnc;
    gd.wsc = d.dns;
    gd.wg = d.dng;
    gd.gs = d.dn_gs;
    gd.a16 = sh.out;
    gd.aexp = sh.exps;
    gd.out = at<float>(ws, l.sh_z);
    const dim3 grid_dn((H + kGemmBN - 1) / kGemmBN, 1);
    const size_t lds_dn = d.wf == FMT_NVFP4 ? (size_t)kGemmBN * (d.S / 16) + 16 : d.wf == FMT_INT4 ? (size_t)kGemmBN * (d.S / 32) + 16 : 16;
    if (d.wf == FMT_FP8)
        hipLaunchKernelGGL((k_grouped_a16<EPI_DOWN, FMT_FP8>), grid_dn, dim3(256), lds_dn, s, gd);
    else if (d.wf == FMT_NVFP4)
        hipLaunchKernelGGL((k_grouped_a16<EPI_DOWN, FMT_NVFP4>), grid_dn, dim3(256), lds_dn, s, gd);
    else
        hipLaunchKernelGGL((k_grouped_a16<EPI_DOWN, FMT_INT4>), grid_dn, dim3(256), lds_dn, s, gd);
    return launched("shared expert down gemm");
}

// Which paths a decode call takes: the routed experts through the grouped
// path, and the shared expert through the grouped GEMMs (the FP8 shared
// expert's small-batch and one-launch forms cover NVFP4 routed experts up
// to kSmallT tokens; the 4-bit shared expert always takes the grouped
// GEMMs).  The small-batch kernels add a shared output in their combine, so
// NVFP4 routed experts keep them up to kSmallT tokens.
struct DecodePlan {
    bool grouped, sh_grouped;
};

DecodePlan decode_plan(const q4moe_experts* ex, int T, bool fp8_shared, bool q4_shared, bool a4, bool force_grouped) {
    DecodePlan p;
    p.sh_grouped = !a4 && (q4_shared || (fp8_shared && (T > kSmallT || ex->fmt != Q4MOE_NVFP4)));
    const bool small_ok = ex->fmt == Q4MOE_NVFP4 && T <= kSmallT;
    p.grouped = force_grouped || (!a4 && w4a16_grouped(ex->fmt, T)) || (p.sh_grouped && !small_ok);
    return p;
}

// The workspace layout of a decode call (as decode_impl plans it).
DecodeWs decode_layout(const q4moe_router* r, const q4moe_experts* ex, const q4moe_shared_fp8* sh,
                       const q4moe_experts* sh4, int32_t n_tok, bool a4 = false, bool grouped = false) {
    const DecodePlan p = decode_plan(ex, n_tok, sh != nullptr, sh4 != nullptr, a4, grouped);
    const int S = sh ? sh->inter : sh4 ? sh4->inter : 0;
    return decode_ws(r->n_experts, ex->hidden, ex->inter, r->top_k, n_tok, S, a4, p.grouped, p.sh_grouped);
}


}  // namespace

// ===========================================================================
// Entry points
// ===========================================================================

extern "C" {

const char* q4moe_status_str(q4moe_status s) {
    switch (s) {
        case Q4MOE_OK: return "ok";
        case Q4MOE_EINVAL: return "invalid argument";
        case Q4MOE_EALIGN: return "misaligned pointer";
        case Q4MOE_EUNSUPPORTED: return "unsupported";
        case Q4MOE_EWORKSPACE: return "workspace too small";
        case Q4MOE_EDEVICE: return "device error";
    }
    return "unknown status";
}

const char* q4moe_last_error(void) { return g_err; }

int32_t q4moe_abi_version(void) { return Q4MOE_ABI_VERSION; }

q4moe_status q4moe_ws_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return fail(Q4MOE_EINVAL, "workspace is NULL");
    if (!aligned(ws, 16) || ws_bytes % 16 != 0)
        return fail(Q4MOE_EALIGN, "workspace must be 16-byte aligned and a multiple of 16 bytes");
    q4moe_status st = device_ready();
    if (st != Q4MOE_OK) return st;
    const size_t n16 = ws_bytes / 16;
    if (n16 == 0) return Q4MOE_OK;
    const size_t blocks = (n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)ws, n16);
    return launched("workspace init");
}

q4moe_status q4moe_ws_check(const void* ws, size_t ws_bytes, void* stream, uint32_t* flags) {
    if (!ws || !flags) return fail(Q4MOE_EINVAL, "workspace / flags is NULL");
    if (ws_bytes < CTRL_WORDS * 4) return fail(Q4MOE_EWORKSPACE, "workspace smaller than its control words");
    q4moe_status st = device_ready();
    if (st != Q4MOE_OK) return st;
    hipError_t e = hipMemcpyAsync(flags, static_cast<const uint32_t*>(ws) + CTRL_FLAGS, 4, hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(Q4MOE_EDEVICE, "reading the workspace status: %s", hipGetErrorString(e));
    return Q4MOE_OK;
}

// --- router ----------------------------------------------------------------

size_t q4moe_router_topk_ws_bytes(const q4moe_router* r, int32_t n_tok) {
    if (!r || n_tok < 1) return 0;
    return router_ws(r->n_experts, r->top_k, n_tok).total;
}

q4moe_status q4moe_router_topk(const q4moe_router* r, const uint16_t* x_bf16, int32_t n_tok, int32_t* ids,
                               float* w, float* logits, void* ws, size_t ws_bytes, void* stream) {
    q4moe_status st = check_router(r);
    if (st != Q4MOE_OK) return st;
    if (n_tok < 1 || n_tok > 65536) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 65536]", n_tok);
    if (!x_bf16 || !ids || !w) return fail(Q4MOE_EINVAL, "x / ids / w is NULL");
    if (!aligned(x_bf16, 16)) return fail(Q4MOE_EALIGN, "x not 16-byte aligned");
    if (!aligned(ids, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4)))
        return fail(Q4MOE_EALIGN, "ids / w / logits not 4-byte aligned");
    RouterWs l = router_ws(r->n_experts, r->top_k, n_tok);
    if ((st = check_ws(ws, ws_bytes, l.total)) != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    return launch_router(router_args(r, x_bf16, n_tok, ws, l, ids, w, logits), (hipStream_t)stream);
}

// --- reference dequantization --------------------------------------------

q4moe_status q4moe_dequant_ref(const q4moe_qmat* m, float* out, void* stream) {
    if (!m) return fail(Q4MOE_EINVAL, "matrix descriptor is NULL");
    if (m->fmt != Q4MOE_NVFP4 && m->fmt != Q4MOE_INT4_G64) return fail(Q4MOE_EINVAL, "unknown format %d", m->fmt);
    const int blk = m->fmt == Q4MOE_NVFP4 ? 16 : 64;
    if (m->rows < 1 || m->cols < blk || m->cols % blk != 0)
        return fail(Q4MOE_EINVAL, "shape %d x %d: rows >= 1 and cols a positive multiple of %d", m->rows, m->cols,
                    blk);
    if (!m->codes || !m->scales || !out) return fail(Q4MOE_EINVAL, "codes / scales / out is NULL");
    if (m->fmt == Q4MOE_NVFP4 && !m->gscale) return fail(Q4MOE_EINVAL, "NVFP4 needs gscale");
    if (m->fmt == Q4MOE_INT4_G64 && m->gscale) return fail(Q4MOE_EINVAL, "INT4_G64 takes no gscale");
    if (!aligned(m->codes, 16) || !aligned(out, 16)) return fail(Q4MOE_EALIGN, "codes / out not 16-byte aligned");
    if (!aligned(m->scales, 4)) return fail(Q4MOE_EALIGN, "scales not 4-byte aligned");
    q4moe_status st = device_ready();
    if (st != Q4MOE_OK) return st;
    const size_t ndw = (size_t)m->rows * m->cols / 8;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       m->fmt, m->rows, m->cols, m->codes, m->scales, m->gscale, out);
    return launched("dequant");
}

// --- W4A16 decode ---------------------------------------------------------

size_t q4moe_w4a16_decode_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    if (!r || !ex || n_tok < 1) return 0;
    return decode_layout(r, ex, nullptr, nullptr, n_tok).total;
}

q4moe_status q4moe_w4a16_decode_taps(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok,
                                     q4moe_decode_taps* out) {
    if (!r || !ex || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    DecodeWs l = decode_layout(r, ex, nullptr, nullptr, n_tok);
    out->y32 = l.y32;
    out->h = l.h;
    return Q4MOE_OK;
}

namespace {

q4moe_status check_shared(const q4moe_shared_fp8* sh, const q4moe_experts* ex, int32_t n_tok) {
    if (!sh) return fail(Q4MOE_EINVAL, "shared expert descriptor is NULL");
    if (sh->hidden != ex->hidden)
        return fail(Q4MOE_EINVAL, "shared expert hidden %d differs from the experts' %d", sh->hidden, ex->hidden);
    if (sh->inter < 64 || sh->inter % 64 != 0 || sh->inter > kMaxDim)
        return fail(Q4MOE_EINVAL, "shared expert inter %d must be a multiple of 64 in [64, %d]", sh->inter, kMaxDim);
    if (!sh->up_codes || !sh->down_codes) return fail(Q4MOE_EINVAL, "shared expert codes are NULL");
    if (!aligned(sh->up_codes, 16) || !aligned(sh->down_codes, 16))
        return fail(Q4MOE_EALIGN, "shared expert codes not 16-byte aligned");
    const float sc[4] = {sh->up_wscale, sh->up_iscale, sh->down_wscale, sh->down_iscale};
    for (float v : sc)
        if (!std::isfinite(v) || v == 0.0f) return fail(Q4MOE_EINVAL, "shared expert scales must be finite and non-zero");
    (void)n_tok;
    return Q4MOE_OK;
}

// The 4-bit W4A16 shared expert: an expert bank of one expert, NVFP4 or
// int4-g64, the routed experts' hidden, inter a multiple of 64.
q4moe_status check_shared_q4(const q4moe_experts* sh, const q4moe_experts* ex) {
    if (!sh) return fail(Q4MOE_EINVAL, "shared expert descriptor is NULL");
    if (sh->n_experts != 1) return fail(Q4MOE_EINVAL, "the shared expert is a bank of one expert (got %d)", sh->n_experts);
    if (sh->fmt != Q4MOE_NVFP4 && sh->fmt != Q4MOE_INT4_G64)
        return fail(Q4MOE_EINVAL, "unknown shared expert format %d", sh->fmt);
    if (sh->hidden != ex->hidden)
        return fail(Q4MOE_EINVAL, "shared expert hidden %d differs from the experts' %d", sh->hidden, ex->hidden);
    if (sh->inter < 64 || sh->inter % 64 != 0 || sh->inter > kMaxDim)
        return fail(Q4MOE_EINVAL, "shared expert inter %d must be a multiple of 64 in [64, %d]", sh->inter, kMaxDim);
    if (!sh->up_codes || !sh->up_scales || !sh->down_codes || !sh->down_scales)
        return fail(Q4MOE_EINVAL, "shared expert code / scale pointer is NULL");
    if (sh->fmt == Q4MOE_NVFP4 && (!sh->up_gscale || !sh->down_gscale))
        return fail(Q4MOE_EINVAL, "an NVFP4 shared expert needs up_gscale and down_gscale");
    if (sh->fmt == Q4MOE_INT4_G64 && (sh->up_gscale || sh->down_gscale))
        return fail(Q4MOE_EINVAL, "an INT4_G64 shared expert takes no per-tensor scale (pass NULL)");
    if (!aligned(sh->up_codes, 16) || !aligned(sh->down_codes, 16))
        return fail(Q4MOE_EALIGN, "shared expert codes not 16-byte aligned");
    if (!aligned(sh->up_scales, 4) || !aligned(sh->down_scales, 4))
        return fail(Q4MOE_EALIGN, "shared expert scales not 4-byte aligned");
    if ((sh->up_gscale && !aligned(sh->up_gscale, 4)) || (sh->down_gscale && !aligned(sh->down_gscale, 4)))
        return fail(Q4MOE_EALIGN, "shared expert gscale not 4-byte aligned");
    return Q4MOE_OK;
}

// a4: the W4A4 single-token decode (activations quantized to NVFP4);
// grouped: the grouped W4A16 path whatever the token count.
q4moe_status decode_impl(const q4moe_router* r, const q4moe_experts* ex, const q4moe_shared_fp8* sh,
                         const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w,
                         void* ws, size_t ws_bytes, void* stream, bool a4 = false, bool force_grouped = false,
                         const q4moe_experts* sh4 = nullptr) {
    q4moe_status st = check_router(r);
    if (st != Q4MOE_OK) return st;
    if ((st = check_experts(ex, r)) != Q4MOE_OK) return st;
    if (n_tok < 1 || n_tok > 65536) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 65536]", n_tok);
    if (sh && (st = check_shared(sh, ex, n_tok)) != Q4MOE_OK) return st;
    if (sh4 && (st = check_shared_q4(sh4, ex)) != Q4MOE_OK) return st;
    if (a4 && ex->fmt != Q4MOE_NVFP4) return fail(Q4MOE_EUNSUPPORTED, "the W4A4 decode takes NVFP4 experts only");
    if (a4 && n_tok > kSmallT8)
        return fail(Q4MOE_EUNSUPPORTED, "the W4A4 decode runs up to %d tokens (n_tok = %d)", kSmallT8, n_tok);
    if (a4 && sh && n_tok > kSmallT)
        return fail(Q4MOE_EUNSUPPORTED, "the W4A4 decode with the shared expert runs up to %d tokens", kSmallT);
    const DecodePlan plan = decode_plan(ex, n_tok, sh != nullptr, sh4 != nullptr, a4, force_grouped);
    if (plan.grouped && (ex->hidden % 64 != 0 || ex->inter % 64 != 0))
        return fail(Q4MOE_EUNSUPPORTED, "the grouped path (and more than %d tokens) needs hidden and inter "
                    "multiples of 64 (got %d, %d)", kSmallT, ex->hidden, ex->inter);
    if (plan.sh_grouped && ex->hidden % 64 != 0)
        return fail(Q4MOE_EUNSUPPORTED, "the shared expert's grouped GEMMs need hidden a multiple of 64 (got %d)",
                    ex->hidden);
    if (!x_bf16 || !y_bf16) return fail(Q4MOE_EINVAL, "x / y is NULL");
    if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16)) return fail(Q4MOE_EALIGN, "x / y not 16-byte aligned");
    if ((ids && !aligned(ids, 4)) || (w && !aligned(w, 4))) return fail(Q4MOE_EALIGN, "ids / w not 4-byte aligned");
    const DecodeWs l = decode_layout(r, ex, sh, sh4, n_tok, a4, force_grouped);
    if ((st = check_ws(ws, ws_bytes, l.total)) != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const float* zsh = nullptr;
    if (plan.sh_grouped) {
        if ((st = launch_shared_grouped(shared_dense(sh, sh4), x_bf16, n_tok, ex->hidden, ws, l, s)) != Q4MOE_OK)
            return st;
        zsh = at<float>(ws, l.sh_z);
    }
    if (plan.grouped) return launch_grouped16(r, ex, x_bf16, n_tok, y_bf16, ids, w, ws, l, s, zsh);

    if (n_tok == 1 && !plan.sh_grouped) {  // one persistent launch for the whole layer
        FusedArgs f;
        f.E = r->n_experts;
        f.H = ex->hidden;
        f.I = ex->inter;
        f.K = r->top_k;
        f.wg = r->w_g;
        f.bias = r->bias;
        f.x = x_bf16;
        f.upc = ex->up_codes;
        f.ups = ex->up_scales;
        f.upg = ex->up_gscale;
        f.dnc = ex->down_codes;
        f.dns = ex->down_scales;
        f.dng = ex->down_gscale;
        f.y = y_bf16;
        f.ids_out = ids;
        f.w_out = w;
        f.ctrl = at<uint32_t>(ws, l.r.ctrl);
        f.sc_tag = at<unsigned long long>(ws, l.sc_tag);
        f.h_tag = at<unsigned long long>(ws, l.h_tag);
        f.z_tag = at<unsigned long long>(ws, l.z_tag);
        f.ids = at<int32_t>(ws, l.r.ids);
        f.w = at<float>(ws, l.r.w);
        f.h = at<float>(ws, l.h);
        f.y32 = at<float>(ws, l.y32);
        f.S = 0;
        f.shu = f.shd = nullptr;
        f.su_w = f.su_in = f.sd_w = f.sd_in = 1.0f;
        f.hq_tag = nullptr;
        f.sh_xq = f.sh_hq = nullptr;
        f.sh_h = nullptr;
        f.xq_codes = f.xq_scales = f.hq_codes = f.hq_scales = nullptr;
        if (a4) {
            f.xq_codes = at<uint8_t>(ws, l.xq_c);
            f.xq_scales = at<uint8_t>(ws, l.xq_s);
            f.hq_codes = at<uint8_t>(ws, l.hq_c);
            f.hq_scales = at<uint8_t>(ws, l.hq_s);
        }
        if (sh) {
            f.S = sh->inter;
            f.shu = sh->up_codes;
            f.shd = sh->down_codes;
            f.su_w = sh->up_wscale;
            f.su_in = sh->up_iscale;
            f.sd_w = sh->down_wscale;
            f.sd_in = sh->down_iscale;
            f.hq_tag = at<unsigned long long>(ws, l.hq_tag);
            f.sh_xq = at<uint8_t>(ws, l.sh_xq);
            f.sh_h = at<float>(ws, l.sh_h);
            f.sh_hq = at<uint8_t>(ws, l.sh_hq);
        }
        // where the single launch does not fit the device and shape, the
        // multi-launch path below takes the token
        if (a4)
            st = sh ? launch_fused<FMT_NVFP4, true, true>(f, s) : launch_fused<FMT_NVFP4, false, true>(f, s);
        else if (sh)
            st = launch_fused<FMT_NVFP4, true, false>(f, s);
        else
            st = ex->fmt == Q4MOE_NVFP4 ? launch_fused<FMT_NVFP4>(f, s) : launch_fused<FMT_INT4>(f, s);
        if (st != Q4MOE_EUNSUPPORTED) return st;
    }

    RouterArgs ra = router_args(r, x_bf16, n_tok, ws, l.r, ids, w, nullptr);
    if (sh && !plan.sh_grouped) {  // the shared expert's own three launches first
        SharedSmallArgs q;
        q.T = n_tok;
        q.H = ex->hidden;
        q.S = sh->inter;
        q.x = x_bf16;
        q.shu = sh->up_codes;
        q.shd = sh->down_codes;
        q.su_w = sh->up_wscale;
        q.su_in = sh->up_iscale;
        q.sd_w = sh->down_wscale;
        q.sd_in = sh->down_iscale;
        q.xq = at<uint8_t>(ws, l.sh_xq);
        q.h = at<float>(ws, l.sh_h);
        q.hq = at<uint8_t>(ws, l.sh_hq);
        q.z = at<float>(ws, l.sh_z);
        const int chu = (q.H / 16 + 63) / 64, chd = (q.S / 16 + 63) / 64;  // 1..4 each
        const dim3 gu((q.S + kShRowsPerWg - 1) / kShRowsPerWg), gd((q.H + kShRowsPerWg - 1) / kShRowsPerWg);
        hipLaunchKernelGGL(k_shared_xcode, dim3((q.T * q.H / 8 + 255) / 256), dim3(256), 0, s, q);
        if ((st = launched("shared expert x codes")) != Q4MOE_OK) return st;
        switch (chu) {
            case 1: hipLaunchKernelGGL(k_shared_up<1>, gu, dim3(256), 0, s, q); break;
            case 2: hipLaunchKernelGGL(k_shared_up<2>, gu, dim3(256), 0, s, q); break;
            case 3: hipLaunchKernelGGL(k_shared_up<3>, gu, dim3(256), 0, s, q); break;
            default: hipLaunchKernelGGL(k_shared_up<4>, gu, dim3(256), 0, s, q); break;
        }
        if ((st = launched("shared expert up")) != Q4MOE_OK) return st;
        switch (chd) {
            case 1: hipLaunchKernelGGL(k_shared_down<1>, gd, dim3(256), 0, s, q); break;
            case 2: hipLaunchKernelGGL(k_shared_down<2>, gd, dim3(256), 0, s, q); break;
            case 3: hipLaunchKernelGGL(k_shared_down<3>, gd, dim3(256), 0, s, q); break;
            default: hipLaunchKernelGGL(k_shared_down<4>, gd, dim3(256), 0, s, q); break;
        }
        if ((st = launched("shared expert down")) != Q4MOE_OK) return st;
        zsh = q.z;
    }
    if (ex->fmt == Q4MOE_NVFP4) {  // each distinct expert streamed once, on MFMA
        // the logits here; the top-k inside the up kernel (one launch fewer)
        hipLaunchKernelGGL(k_router_logits, dim3(ra.E, (ra.T + 3) / 4), dim3(256), 0, s, ra);
        if ((st = launched("router logits")) != Q4MOE_OK) return st;
        SmallMoeArgs b;
        b.E = ex->n_experts;
        b.H = ex->hidden;
        b.I = ex->inter;
        b.K = r->top_k;
        b.T = n_tok;
        b.upc = ex->up_codes;
        b.ups = static_cast<const uint8_t*>(ex->up_scales);
        b.upg = ex->up_gscale;
        b.dnc = ex->down_codes;
        b.dns = static_cast<const uint8_t*>(ex->down_scales);
        b.dng = ex->down_gscale;
        b.x = x_bf16;
        b.ids = ra.ids;
        b.w = ra.w;
        b.h = at<float>(ws, l.h);
        b.zw = at<float>(ws, l.zw);
        b.y32 = at<float>(ws, l.y32);
        b.y = y_bf16;
        b.ra = ra;
        b.zsh = zsh;
        b.xq_codes = a4 ? at<uint8_t>(ws, l.xq_c) : nullptr;
        b.xq_scales = a4 ? at<uint8_t>(ws, l.xq_s) : nullptr;
        b.hq_codes = a4 ? at<uint8_t>(ws, l.hq_c) : nullptr;
        b.hq_scales = a4 ? at<uint8_t>(ws, l.hq_s) : nullptr;
        return launch_small(b, a4, s);
    }
    if ((st = launch_router(ra, s)) != Q4MOE_OK) return st;

    MoeArgs a;
    a.fmt = ex->fmt;
    a.E = ex->n_experts;
    a.H = ex->hidden;
    a.I = ex->inter;
    a.K = r->top_k;
    a.T = n_tok;
    a.upc = ex->up_codes;
    a.ups = ex->up_scales;
    a.upg = ex->up_gscale;
    a.dnc = ex->down_codes;
    a.dns = ex->down_scales;
    a.dng = ex->down_gscale;
    a.x = x_bf16;
    a.ids = ra.ids;
    a.w = ra.w;
    a.h = at<float>(ws, l.h);
    a.y32 = at<float>(ws, l.y32);
    a.y = y_bf16;
    if (ex->fmt == Q4MOE_NVFP4) {
        if ((st = launch_up<FMT_NVFP4>(a, s)) != Q4MOE_OK) return st;
        return launch_down<FMT_NVFP4>(a, s);
    }
    if ((st = launch_up<FMT_INT4>(a, s)) != Q4MOE_OK) return st;
    return launch_down<FMT_INT4>(a, s);
}

}  // namespace

q4moe_status q4moe_w4a16_decode(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                                int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* ws,
                                size_t ws_bytes, void* stream) {
    return decode_impl(r, ex, nullptr, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream);
}

size_t q4moe_w4a16_decode_stack_ws_bytes(const q4moe_router* r, const q4moe_experts* ex) {
    return q4moe_w4a16_decode_ws_bytes(r, ex, 1);
}

q4moe_status q4moe_w4a16_decode_stack(const q4moe_router* routers, const q4moe_experts* experts, int32_t n_layers,
                                      const uint16_t* const* x_bf16, uint16_t* const* y_bf16, int32_t chain,
                                      int32_t* const* ids, float* const* w, void* ws, size_t ws_bytes,
                                      void* stream) {
    if (!routers || !experts || !x_bf16 || !y_bf16) return fail(Q4MOE_EINVAL, "routers / experts / x / y is NULL");
    if (n_layers < 1 || n_layers > 4096) return fail(Q4MOE_EINVAL, "n_layers %d outside [1, 4096]", n_layers);
    const q4moe_router* r0 = &routers[0];
    const q4moe_experts* e0 = &experts[0];
    q4moe_status st;
    for (int l = 0; l < n_layers; ++l) {
        const q4moe_router* r = &routers[l];
        const q4moe_experts* ex = &experts[l];
        if ((st = check_router(r)) != Q4MOE_OK || (st = check_experts(ex, r)) != Q4MOE_OK) return st;
        if (r->n_experts != r0->n_experts || r->hidden != r0->hidden || r->top_k != r0->top_k ||
            ex->inter != e0->inter || ex->fmt != e0->fmt)
            return fail(Q4MOE_EINVAL, "layer %d's shape or format differs from layer 0's", l);
        const uint16_t* x = x_bf16[l];
        if (!(chain && l > 0) && (!x || !aligned(x, 16)))
            return fail(x ? Q4MOE_EALIGN : Q4MOE_EINVAL, "x of layer %d is NULL or not 16-byte aligned", l);
        if (!y_bf16[l] || !aligned(y_bf16[l], 16))
            return fail(y_bf16[l] ? Q4MOE_EALIGN : Q4MOE_EINVAL, "y of layer %d is NULL or not 16-byte aligned", l);
        if ((ids && ids[l] && !aligned(ids[l], 4)) || (w && w[l] && !aligned(w[l], 4)))
            return fail(Q4MOE_EALIGN, "ids / w of layer %d not 4-byte aligned", l);
    }
    const DecodeWs lay = decode_layout(r0, e0, nullptr, nullptr, 1);
    if ((st = check_ws(ws, ws_bytes, lay.total)) != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    StackArgs sa{};
    FusedArgs& f = sa.a;
    f.E = r0->n_experts;
    f.H = e0->hidden;
    f.I = e0->inter;
    f.K = r0->top_k;
    f.ctrl = at<uint32_t>(ws, lay.r.ctrl);
    f.sc_tag = at<unsigned long long>(ws, lay.sc_tag);
    f.h_tag = at<unsigned long long>(ws, lay.h_tag);
    f.z_tag = at<unsigned long long>(ws, lay.z_tag);
    f.ids = at<int32_t>(ws, lay.r.ids);
    f.w = at<float>(ws, lay.r.w);
    f.h = at<float>(ws, lay.h);
    f.y32 = at<float>(ws, lay.y32);
    f.su_w = f.su_in = f.sd_w = f.sd_in = 1.0f;
    sa.y_tag = at<unsigned long long>(ws, lay.y_tag);
    sa.done_tag = at<unsigned long long>(ws, lay.done_tag);
    sa.chain = chain ? 1 : 0;
    // one launch per kStackMax layers; the first layer of a later launch
    // reads the previous layer's y from memory (the launches are in order)
    for (int l0 = 0; l0 < n_layers; l0 += kStackMax) {
        const int n = std::min(kStackMax, n_layers - l0);
        sa.n_layers = n;
        for (int i = 0; i < n; ++i) {
            const int l = l0 + i;
            const q4moe_router* r = &routers[l];
            const q4moe_experts* ex = &experts[l];
            StackLayer& L = sa.layer[i];
            L.wg = r->w_g;
            L.bias = r->bias;
            L.x = chain && l > 0 ? (i == 0 ? y_bf16[l - 1] : nullptr) : x_bf16[l];
            L.upc = ex->up_codes;
            L.ups = ex->up_scales;
            L.upg = ex->up_gscale;
            L.dnc = ex->down_codes;
            L.dns = ex->down_scales;
            L.dng = ex->down_gscale;
            L.y = y_bf16[l];
            L.ids_out = ids ? ids[l] : nullptr;
            L.w_out = w ? w[l] : nullptr;
        }
        st = e0->fmt == Q4MOE_NVFP4 ? launch_stack<FMT_NVFP4>(sa, s) : launch_stack<FMT_INT4>(sa, s);
        if (st == Q4MOE_EUNSUPPORTED) {
            // a shape or device the one launch does not fit: one call per
            // layer, in the same order and with the same results
            for (int i = 0; i < n; ++i) {
                const int l = l0 + i;
                const uint16_t* x = chain && l > 0 ? y_bf16[l - 1] : x_bf16[l];
                st = decode_impl(&routers[l], &experts[l], nullptr, x, 1, y_bf16[l], ids ? ids[l] : nullptr,
                                 w ? w[l] : nullptr, ws, ws_bytes, stream);
                if (st != Q4MOE_OK) return st;
            }
        } else if (st != Q4MOE_OK) {
            return st;
        }
    }
    return Q4MOE_OK;
}

size_t q4moe_w4a16_grouped_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    if (!r || !ex || n_tok < 1) return 0;
    return decode_layout(r, ex, nullptr, nullptr, n_tok, false, true).total;
}

q4moe_status q4moe_w4a16_grouped(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                                 int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* ws,
                                 size_t ws_bytes, void* stream) {
    return decode_impl(r, ex, nullptr, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream, false, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode without a caller workspace: its workspace is a file-scope
// device array, one copy per GPU, zero-filled when the code object is
// loaded and kept until the process ends.  Its device address on each GPU
// is looked up once (with that GPU current) and used from then on; the
// array's name in host code is only a stand-in for the symbol.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = 7u << 19;  // 3.5 MiB: the prefix (~2.5 MB) plus room for 1-4 tokens
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

q4moe_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(Q4MOE_EDEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(Q4MOE_EDEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(Q4MOE_EDEVICE, "static scratch address on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return Q4MOE_OK;
}

}  // namespace

extern "C" {

q4moe_status q4moe_w4a16_decode_noalloc(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                                        int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* stream) {
    q4moe_status st = check_router(r);
    if (st != Q4MOE_OK) return st;
    if ((st = check_experts(ex, r)) != Q4MOE_OK) return st;
    if (n_tok < 1 || n_tok > 4) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 4]", n_tok);
    const size_t need =
        decode_layout(r, ex, nullptr, nullptr, n_tok).total;
    if (need > kNoAllocScratchBytes)
        return fail(Q4MOE_EWORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu", need,
                    kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != Q4MOE_OK) return st;
    return decode_impl(r, ex, nullptr, x_bf16, n_tok, y_bf16, ids, w, ws, kNoAllocScratchBytes, stream);
}

size_t q4moe_w4a16_decode_shared_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                          const q4moe_shared_fp8* sh, int32_t n_tok) {
    if (!r || !ex || !sh || n_tok < 1) return 0;
    return decode_layout(r, ex, sh, nullptr, n_tok).total;
}

q4moe_status q4moe_w4a16_decode_shared(const q4moe_router* r, const q4moe_experts* ex,
                                       const q4moe_shared_fp8* sh, const uint16_t* x_bf16, int32_t n_tok,
                                       uint16_t* y_bf16, int32_t* ids, float* w, void* ws, size_t ws_bytes,
                                       void* stream) {
    if (!sh) return fail(Q4MOE_EINVAL, "shared expert descriptor is NULL");
    return decode_impl(r, ex, sh, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream);
}

size_t q4moe_w4a16_decode_shared_q4_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                             const q4moe_experts* sh, int32_t n_tok) {
    if (!r || !ex || !sh || n_tok < 1) return 0;
    return decode_layout(r, ex, nullptr, sh, n_tok).total;
}

q4moe_status q4moe_w4a16_decode_shared_q4(const q4moe_router* r, const q4moe_experts* ex, const q4moe_experts* sh,
                                          const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16, int32_t* ids,
                                          float* w, void* ws, size_t ws_bytes, void* stream) {
    if (!sh) return fail(Q4MOE_EINVAL, "shared expert descriptor is NULL");
    return decode_impl(r, ex, nullptr, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream, false, false, sh);
}

q4moe_status q4moe_w4a16_decode_shared_q4_taps(const q4moe_router* r, const q4moe_experts* ex,
                                               const q4moe_experts* sh, int32_t n_tok, q4moe_shared_taps* out) {
    if (!r || !ex || !sh || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    DecodeWs l = decode_layout(r, ex, nullptr, sh, n_tok);
    out->y32 = l.y32;
    out->h = l.h;
    out->xq = 0;
    out->sh_h32 = l.sh_h;
    out->sh_hq = 0;
    return Q4MOE_OK;
}

size_t q4moe_w4a4_decode_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    if (!r || !ex || n_tok < 1) return 0;
    return decode_layout(r, ex, nullptr, nullptr, n_tok, true).total;
}

q4moe_status q4moe_w4a4_decode(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                               int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* ws,
                               size_t ws_bytes, void* stream) {
    return decode_impl(r, ex, nullptr, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream, true);
}

q4moe_status q4moe_w4a4_decode_taps(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok,
                                    q4moe_w4a4_token_taps* out) {
    if (!r || !ex || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    DecodeWs l = decode_layout(r, ex, nullptr, nullptr, n_tok, true);
    out->y32 = l.y32;
    out->h32 = l.h;
    out->xq_codes = l.xq_c;
    out->xq_scales = l.xq_s;
    out->hq_codes = l.hq_c;
    out->hq_scales = l.hq_s;
    return Q4MOE_OK;
}

size_t q4moe_w4a4_decode_shared_ws_bytes(const q4moe_router* r, const q4moe_experts* ex,
                                         const q4moe_shared_fp8* sh, int32_t n_tok) {
    if (!r || !ex || !sh || n_tok < 1) return 0;
    return decode_layout(r, ex, sh, nullptr, n_tok, true).total;
}

q4moe_status q4moe_w4a4_decode_shared(const q4moe_router* r, const q4moe_experts* ex, const q4moe_shared_fp8* sh,
                                      const uint16_t* x_bf16, int32_t n_tok, uint16_t* y_bf16, int32_t* ids,
                                      float* w, void* ws, size_t ws_bytes, void* stream) {
    if (!sh) return fail(Q4MOE_EINVAL, "shared expert descriptor is NULL");
    return decode_impl(r, ex, sh, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream, true);
}

q4moe_status q4moe_w4a4_decode_shared_taps(const q4moe_router* r, const q4moe_experts* ex,
                                           const q4moe_shared_fp8* sh, int32_t n_tok, q4moe_w4a4_shared_taps* out) {
    if (!r || !ex || !sh || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    DecodeWs l = decode_layout(r, ex, sh, nullptr, n_tok, true);
    out->y32 = l.y32;
    out->h32 = l.h;
    out->xq_codes = l.xq_c;
    out->xq_scales = l.xq_s;
    out->hq_codes = l.hq_c;
    out->hq_scales = l.hq_s;
    out->sh_xq = l.sh_xq;
    out->sh_h32 = l.sh_h;
    out->sh_hq = l.sh_hq;
    return Q4MOE_OK;
}

size_t q4moe_quantize_weights_ws_bytes(int32_t rows, int32_t cols) {
    (void)rows;
    (void)cols;
    return kPrefixBytes + (size_t)kWqMaxBlocks * sizeof(float);
}

q4moe_status q4moe_quantize_weights(const uint16_t* w_bf16, int32_t rows, int32_t cols, int32_t mode,
                                    uint8_t* codes, uint8_t* scales, float* gscale, void* ws, size_t ws_bytes,
                                    void* stream) {
    if (!w_bf16 || !codes || !scales || !gscale) return fail(Q4MOE_EINVAL, "w / codes / scales / gscale is NULL");
    if (rows < 1 || cols < 16 || cols % 16 != 0 || (long long)rows * cols > (1LL << 34))
        return fail(Q4MOE_EINVAL, "shape %d x %d: rows >= 1, cols a positive multiple of 16, at most 2^34 weights",
                    rows, cols);
    if (mode != Q4MOE_WQ_MAX && mode != Q4MOE_WQ_MSE) return fail(Q4MOE_EINVAL, "unknown scale mode %d", mode);
    if (!aligned(w_bf16, 16) || !aligned(codes, 8) || !aligned(gscale, 4))
        return fail(Q4MOE_EALIGN, "w not 16-byte, codes not 8-byte or gscale not 4-byte aligned");
    q4moe_status st = check_ws(ws, ws_bytes, q4moe_quantize_weights_ws_bytes(rows, cols));
    if (st != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t n8 = (size_t)rows * cols / 8, nblocks = (size_t)rows * cols / 16;
    const int grid1 = (int)std::min<size_t>(kWqMaxBlocks, (n8 + 255) / 256);
    float* partial = at<float>(ws, kPrefixBytes);
    hipLaunchKernelGGL(k_wq_amax, dim3(grid1), dim3(256), 0, s, reinterpret_cast<const uint4*>(w_bf16), n8, partial);
    if ((st = launched("weight quantizer maximum")) != Q4MOE_OK) return st;
    WqArgs a;
    a.w = reinterpret_cast<const uint4*>(w_bf16);
    a.nblocks = nblocks;
    a.partial = partial;
    a.npartial = grid1;
    a.mse = mode;
    a.codes = codes;
    a.scales = scales;
    a.gscale = gscale;
    const dim3 grid2((unsigned)((nblocks + 255) / 256));
    if (mode == Q4MOE_WQ_MSE)
        hipLaunchKernelGGL(k_wq_quant<true>, grid2, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_wq_quant<false>, grid2, dim3(256), 0, s, a);
    return launched("weight quantizer");
}

size_t q4moe_w4a4_moe_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    if (!r || !ex || n_tok < 1) return 0;
    const size_t small = decode_layout(r, ex, nullptr, nullptr, 1, true).total;
    const size_t grouped = w4a4_ws(r->n_experts, ex->hidden, ex->inter, r->top_k, n_tok).total;
    return std::max(small, grouped);
}

q4moe_status q4moe_w4a4_moe(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16, int32_t n_tok,
                            uint16_t* y_bf16, int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
    q4moe_status st = check_w4a4(r, ex, n_tok);
    if (st != Q4MOE_OK) return st;
    if (!x_bf16 || !y_bf16 || !ids || !w) return fail(Q4MOE_EINVAL, "x / y / ids / w is NULL");
    if ((st = check_ws(ws, ws_bytes, q4moe_w4a4_moe_ws_bytes(r, ex, n_tok))) != Q4MOE_OK) return st;
    if (n_tok <= Q4MOE_W4A4_PER_TOKEN_MAX_TOKENS) {
        // one single-token launch per token, in order on the stream (each
        // call advances the workspace's epoch, so the calls can share it);
        // measured cold at the full shapes, these beat the one-pass
        // small-batch kernels (2 tokens: 34 us against 50 us) and the grouped
        // pipeline up to 7 tokens
        const size_t H = (size_t)ex->hidden, K = (size_t)r->top_k;
        for (int32_t t = 0; t < n_tok; ++t) {
            st = decode_impl(r, ex, nullptr, x_bf16 + t * H, 1, y_bf16 + t * H, ids + t * K, w + t * K, ws, ws_bytes,
                             stream, true);
            if (st != Q4MOE_OK) return st;
        }
        return st;
    }
    return q4moe_w4a4_grouped(r, ex, x_bf16, n_tok, y_bf16, ids, w, ws, ws_bytes, stream);
}

q4moe_status q4moe_w4a16_decode_shared_taps(const q4moe_router* r, const q4moe_experts* ex,
                                            const q4moe_shared_fp8* sh, int32_t n_tok, q4moe_shared_taps* out) {
    if (!r || !ex || !sh || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    DecodeWs l = decode_layout(r, ex, sh, nullptr, n_tok);
    out->y32 = l.y32;
    out->h = l.h;
    out->xq = l.sh_xq;
    out->sh_h32 = l.sh_h;
    out->sh_hq = l.sh_hq;
    return Q4MOE_OK;
}

// --- W4A4 grouped -----------------------------------------------------------

size_t q4moe_w4a4_grouped_ws_bytes(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok) {
    if (!r || !ex || n_tok < 1) return 0;
    return w4a4_ws(r->n_experts, ex->hidden, ex->inter, r->top_k, n_tok).total;
}

q4moe_status q4moe_w4a4_grouped_taps(const q4moe_router* r, const q4moe_experts* ex, int32_t n_tok,
                                     q4moe_w4a4_taps* out) {
    if (!r || !ex || !out || n_tok < 1) return fail(Q4MOE_EINVAL, "NULL descriptor or n_tok < 1");
    W4a4Ws l = w4a4_ws(r->n_experts, ex->hidden, ex->inter, r->top_k, n_tok);
    out->perm = l.perm;
    out->expert_offsets = l.offsets;
    out->xq_codes = l.xq_codes;
    out->xq_scales = l.xq_scales;
    out->h32 = l.h32;
    out->hq_codes = l.hq_codes;
    out->hq_scales = l.hq_scales;
    out->y32 = l.y32;
    return Q4MOE_OK;
}

q4moe_status q4moe_w4a4_grouped(const q4moe_router* r, const q4moe_experts* ex, const uint16_t* x_bf16,
                                int32_t n_tok, uint16_t* y_bf16, int32_t* ids, float* w, void* ws,
                                size_t ws_bytes, void* stream) {
    q4moe_status st = check_w4a4(r, ex, n_tok);
    if (st != Q4MOE_OK) return st;
    if (!x_bf16 || !y_bf16 || !ids || !w) return fail(Q4MOE_EINVAL, "x / y / ids / w is NULL");
    if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16)) return fail(Q4MOE_EALIGN, "x / y not 16-byte aligned");
    if (!aligned(ids, 4) || !aligned(w, 4)) return fail(Q4MOE_EALIGN, "ids / w not 4-byte aligned");
    const int E = r->n_experts, H = ex->hidden, I = ex->inter, K = r->top_k, T = n_tok;
    W4a4Ws l = w4a4_ws(E, H, I, K, T);
    if ((st = check_ws(ws, ws_bytes, l.total)) != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t rows = (size_t)T * K;

    // router
    RouterArgs ra = router_args(r, x_bf16, T, ws, l.r, ids, w, nullptr);
    launch_router_gemm(ra, s);
    if ((st = launched("router gemm")) != Q4MOE_OK) return st;
    hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, ra);
    if ((st = launched("router top-k")) != Q4MOE_OK) return st;

    // dispatch
    DispatchArgs da;
    da.ids = ra.ids;
    da.T = T;
    da.K = K;
    da.E = E;
    da.counts = at<int32_t>(ws, l.counts);
    da.lists = at<int32_t>(ws, l.lists);
    da.offsets = at<int32_t>(ws, l.offsets);
    da.perm = at<int32_t>(ws, l.perm);
    da.inv = at<int32_t>(ws, l.inv);
    da.act = nullptr;
    da.n_act = nullptr;
    hipLaunchKernelGGL(k_dispatch, dim3(E), dim3(64), 0, s, da);
    if ((st = launched("dispatch")) != Q4MOE_OK) return st;
    hipLaunchKernelGGL(k_dispatch_scan, dim3(E), dim3(256), 0, s, da);
    if ((st = launched("dispatch scan")) != Q4MOE_OK) return st;

    // x -> NVFP4
    QuantArgs qx;
    qx.rows = T;
    qx.cols = H;
    qx.v = x_bf16;
    qx.codes = at<uint8_t>(ws, l.xq_codes);
    qx.scales = at<uint8_t>(ws, l.xq_scales);
    const size_t nbx = (size_t)T * H / 16;  // one 16-block per lane
    hipLaunchKernelGGL((k_quant_nvfp4<true>), dim3((unsigned)((nbx + 255) / 256)), dim3(256), 0, s, qx);
    if ((st = launched("x quantization")) != Q4MOE_OK) return st;

    // up: h = relu(g u)^2
    GemmArgs gu;
    gu.N = I;
    gu.Kd = H;
    gu.wc = ex->up_codes;
    gu.wsc = static_cast<const uint8_t*>(ex->up_scales);
    gu.wg = ex->up_gscale;
    gu.ac = qx.codes;
    gu.asc = qx.scales;
    gu.offsets = da.offsets;
    gu.perm = da.perm;
    gu.K = K;
    gu.a_by_token = 1;
    gu.out = at<float>(ws, l.h32);
    hipLaunchKernelGGL((k_grouped_gemm<EPI_UP>), dim3((I + kGemmBN - 1) / kGemmBN, E), dim3(256),
                       (size_t)kGemmBN * (H / 16) + 16, s, gu);
    if ((st = launched("grouped up gemm")) != Q4MOE_OK) return st;

    // h -> NVFP4
    QuantArgs qh;
    qh.rows = (int)rows;
    qh.cols = I;
    qh.v = gu.out;
    qh.codes = at<uint8_t>(ws, l.hq_codes);
    qh.scales = at<uint8_t>(ws, l.hq_scales);
    const size_t nbh = rows * I / 16;  // one 16-block per lane
    hipLaunchKernelGGL((k_quant_nvfp4<false>), dim3((unsigned)((nbh + 255) / 256)), dim3(256), 0, s, qh);
    if ((st = launched("h quantization")) != Q4MOE_OK) return st;

    // down: g z per (token, slot) row (the gate is applied in the combine)
    GemmArgs gd = gu;
    gd.N = H;
    gd.Kd = I;
    gd.wc = ex->down_codes;
    gd.wsc = static_cast<const uint8_t*>(ex->down_scales);
    gd.wg = ex->down_gscale;
    gd.ac = qh.codes;
    gd.asc = qh.scales;
    gd.a_by_token = 0;
    gd.out = at<float>(ws, l.z);
    hipLaunchKernelGGL((k_grouped_gemm<EPI_DOWN>), dim3((H + kGemmBN - 1) / kGemmBN, E), dim3(256),
                       (size_t)kGemmBN * (I / 16) + 16, s, gd);
    if ((st = launched("grouped down gemm")) != Q4MOE_OK) return st;

    // combine
    // one workgroup per token, 4 columns per lane (H % 64 == 0, H <= 4096)
    hipLaunchKernelGGL(k_combine, dim3((unsigned)T), dim3((unsigned)((H / 4 + 63) / 64 * 64)), 0, s, T, K, H, da.inv, ra.w,
                       gd.out, at<float>(ws, l.y32), y_bf16);
    return launched("combine");
}

// --- lm_head GEMV ---------------------------------------------------------

size_t q4moe_w4a16_gemv_ws_bytes(const q4moe_qmat* m, int32_t n_tok) {
    if (!m || n_tok < 1) return 0;
    return gemv_ws(n_tok).total;
}

q4moe_status q4moe_w4a16_gemv(const q4moe_qmat* m, const uint16_t* x_bf16, int32_t n_tok, float* logits,
                              int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
    if (!m) return fail(Q4MOE_EINVAL, "matrix descriptor is NULL");
    if (m->fmt != Q4MOE_NVFP4) return fail(Q4MOE_EUNSUPPORTED, "the lm_head GEMV takes NVFP4 only");
    if (m->rows < 1 || m->cols < 32 || m->cols % 32 != 0 || m->cols > kMaxDim)
        return fail(Q4MOE_EINVAL, "shape %d x %d: cols a multiple of 32 in [32, %d]", m->rows, m->cols, kMaxDim);
    if (n_tok < 1 || n_tok > 4) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 4]", n_tok);
    if ((uint64_t)m->rows * (uint64_t)(m->cols / 2) > 0xFFFFFFFFull)
        return fail(Q4MOE_EUNSUPPORTED, "lm_head codes of %d x %d exceed 4 GiB", m->rows, m->cols);
    if (!m->codes || !m->scales || !m->gscale || !x_bf16 || !logits)
        return fail(Q4MOE_EINVAL, "codes / scales / gscale / x / logits is NULL");
    if (!aligned(m->codes, 16) || !aligned(x_bf16, 16) || !aligned(logits, 16))
        return fail(Q4MOE_EALIGN, "codes / x / logits not 16-byte aligned");
    if (!aligned(m->scales, 4) || (argmax && !aligned(argmax, 4)))
        return fail(Q4MOE_EALIGN, "scales / argmax not 4-byte aligned");
    GemvWs l = gemv_ws(n_tok);
    q4moe_status st = check_ws(ws, ws_bytes, l.total);
    if (st != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    GemvArgs a;
    a.rows = m->rows;
    a.cols = m->cols;
    a.T = n_tok;
    a.codes = m->codes;
    a.scales = static_cast<const uint8_t*>(m->scales);
    a.gscale = m->gscale;
    a.x = x_bf16;
    a.logits = logits;
    a.argmax = argmax;
    a.keys = at<unsigned long long>(ws, l.keys);
    hipStream_t s = (hipStream_t)stream;
    const int nj = (m->cols + 127) / 128;  // 128-column pieces per row: 1..32
    const int groups = (m->rows + 15) / 16;
    // NJ: exact for the 2688-wide lm_head, else the next multiple of 4
    const int NJ = nj == 21 ? 21 : (nj + 3) / 4 * 4;
    int grid = 0;
#define Q4_GEMV(JJ, TT)                                                                              \
    do {                                                                                             \
        grid = persistent_grid(k_gemv_mfma<JJ, TT>, 256, std::min((groups + 3) / 4, kMaxGemvBlocks)); \
        if (grid < 1) return fail(Q4MOE_EDEVICE, "occupancy query failed");                          \
        hipLaunchKernelGGL((k_gemv_mfma<JJ, TT>), dim3(grid), dim3(256), 0, s, a);                   \
    } while (0)
#define Q4_GEMV_T(JJ)                  \
    switch (n_tok) {                   \
        case 1: Q4_GEMV(JJ, 1); break; \
        case 2: Q4_GEMV(JJ, 2); break; \
        case 3: Q4_GEMV(JJ, 3); break; \
        default: Q4_GEMV(JJ, 4); break; \
    }
    switch (NJ) {
        case 4: Q4_GEMV_T(4); break;
        case 8: Q4_GEMV_T(8); break;
        case 12: Q4_GEMV_T(12); break;
        case 16: Q4_GEMV_T(16); break;
        case 20: Q4_GEMV_T(20); break;
        case 21: Q4_GEMV_T(21); break;
        case 24: Q4_GEMV_T(24); break;
        case 28: Q4_GEMV_T(28); break;
        default: Q4_GEMV_T(32); break;
    }
#undef Q4_GEMV_T
#undef Q4_GEMV
    if ((st = launched("lm_head gemv")) != Q4MOE_OK) return st;
    if (argmax) {
        hipLaunchKernelGGL(k_argmax_reduce, dim3(1), dim3(256), 0, s, a.keys, grid, n_tok, argmax);
        return launched("lm_head argmax");
    }
    return Q4MOE_OK;
}


// --- FP8 W8A8 GEMV (the drafter's lm_head) ---------------------------------

size_t q4moe_fp8_gemv_ws_bytes(const q4moe_fp8_mat* m, int32_t n_tok) {
    if (!m || n_tok < 1 || m->cols < 1) return 0;
    return fp8_gemv_ws(n_tok, m->cols).total;
}

q4moe_status q4moe_fp8_gemv_taps(const q4moe_fp8_mat* m, int32_t n_tok, size_t* xq) {
    if (!m || !xq || n_tok < 1 || m->cols < 1) return fail(Q4MOE_EINVAL, "NULL argument or n_tok < 1");
    *xq = fp8_gemv_ws(n_tok, m->cols).xq;
    return Q4MOE_OK;
}

q4moe_status q4moe_fp8_gemv(const q4moe_fp8_mat* m, const uint16_t* x_bf16, int32_t n_tok, float* logits,
                            int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
    if (!m) return fail(Q4MOE_EINVAL, "matrix descriptor is NULL");
    if (m->rows < 1 || m->cols < 64 || m->cols % 64 != 0 || m->cols > kMaxDim)
        return fail(Q4MOE_EINVAL, "shape %d x %d: cols a multiple of 64 in [64, %d]", m->rows, m->cols, kMaxDim);
    if (n_tok < 1 || n_tok > 4) return fail(Q4MOE_EINVAL, "n_tok %d outside [1, 4]", n_tok);
    if ((uint64_t)m->rows * (uint64_t)m->cols > 0xFFFFFFFFull)
        return fail(Q4MOE_EUNSUPPORTED, "FP8 codes of %d x %d exceed 4 GiB", m->rows, m->cols);
    if (!std::isfinite(m->wscale) || !std::isfinite(m->iscale) || m->wscale == 0.0f || m->iscale == 0.0f)
        return fail(Q4MOE_EINVAL, "wscale / iscale must be finite and non-zero");
    if (!m->codes || !x_bf16 || !logits) return fail(Q4MOE_EINVAL, "codes / x / logits is NULL");
    if (!aligned(m->codes, 16) || !aligned(x_bf16, 16) || !aligned(logits, 16))
        return fail(Q4MOE_EALIGN, "codes / x / logits not 16-byte aligned");
    if (argmax && !aligned(argmax, 4)) return fail(Q4MOE_EALIGN, "argmax not 4-byte aligned");
    Fp8GemvWs l = fp8_gemv_ws(n_tok, m->cols);
    q4moe_status st = check_ws(ws, ws_bytes, l.total);
    if (st != Q4MOE_OK) return st;
    if ((st = device_ready()) != Q4MOE_OK) return st;
    Fp8GemvArgs a;
    a.rows = m->rows;
    a.cols = m->cols;
    a.T = n_tok;
    a.codes = m->codes;
    a.wscale = m->wscale;
    a.iscale = m->iscale;
    a.x = x_bf16;
    a.logits = logits;
    a.xq = at<uint8_t>(ws, l.xq);
    a.keys = at<unsigned long long>(ws, l.keys);
    hipStream_t s = (hipStream_t)stream;
    const int nj = m->cols / 64;  // 64-column pieces per row: 1..64
    const int groups = (m->rows + 15) / 16;
    // NJ8: exact for the 2688-wide lm_head, else 16, 32, 48 or 64
    const int NJ8 = nj == 42 ? 42 : (nj + 15) / 16 * 16;
    int grid = 0;
#define Q4_GEMV8(JJ, TT)                                                                             \
    do {                                                                                             \
        grid = persistent_grid(k_gemv_fp8<JJ, TT>, 256, std::min((groups + 3) / 4, kMaxGemvBlocks));  \
        if (grid < 1) return fail(Q4MOE_EDEVICE, "occupancy query failed");                          \
        hipLaunchKernelGGL((k_gemv_fp8<JJ, TT>), dim3(grid), dim3(256), 0, s, a);                    \
    } while (0)
#define Q4_GEMV8_T(JJ)                  \
    switch (n_tok) {                    \
        case 1: Q4_GEMV8(JJ, 1); break; \
        case 2: Q4_GEMV8(JJ, 2); break; \
        case 3: Q4_GEMV8(JJ, 3); break; \
        default: Q4_GEMV8(JJ, 4); break; \
    }
    switch (NJ8) {
        case 16: Q4_GEMV8_T(16); break;
        case 32: Q4_GEMV8_T(32); break;
        case 42: Q4_GEMV8_T(42); break;
        case 48: Q4_GEMV8_T(48); break;
        default: Q4_GEMV8_T(64); break;
    }
#undef Q4_GEMV8_T
#undef Q4_GEMV8
    if ((st = launched("fp8 gemv")) != Q4MOE_OK) return st;
    if (argmax) {
        hipLaunchKernelGGL(k_argmax_reduce, dim3(1), dim3(256), 0, s, a.keys, grid, n_tok, argmax);
        return launched("fp8 gemv argmax");
    }
    return Q4MOE_OK;
}

}  // extern "C"
