// Measurement build (libq4moe_probe.so): the whole library with per-workgroup
// phase timestamps in the one-launch decode, plus three reference kernels, for
// the floor measurements of gemm_router_fp32_amd/floor_probe.py.  Nothing in
// the library, the tests or the benchmark's timed region loads it.
//
// Phase marks: at each Q4MOE_PHASE(i) of k_decode_fused thread 0 of every
// workgroup records s_memrealtime (100 MHz) in LDS; at the end it writes the
// workgroup's marks, its per-wave marks (Q4MOE_WAVE_MARK) and the shader
// clock ticks (s_memtime) at the start and the end to slot (n % 32) of a
// device table, n being the number of layers the workgroup has run before
// (its own count, so that in a stacked launch, where workgroups pass from one
// layer to the next at different times, every layer keeps its own slot).
// The marks add a few instructions per phase and one 48-word store per
// workgroup; they change no data path.
#include <hip/hip_runtime.h>

constexpr int kProbeSlots = 32, kProbeWgs = 256, kProbeWords = 48;
__device__ unsigned long long q4p_buf[kProbeSlots][kProbeWgs][kProbeWords];
__device__ unsigned int q4p_count[kProbeWgs];  // layers run, per workgroup
__shared__ unsigned long long q4p_wlds[8][4];

__device__ __forceinline__ void q4p_wave(int i) {
    if ((threadIdx.x & 63) == 0) q4p_wlds[threadIdx.x >> 6][i] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void q4p_mark(int i) {
    __shared__ unsigned long long q4p_lds[16];
    __shared__ unsigned int q4p_slot;
    if (i == 10) __syncthreads();  // the end: every wave of the workgroup
    if (threadIdx.x == 0) {
        if (i == 0) {
            q4p_slot = (blockIdx.x < kProbeWgs ? q4p_count[blockIdx.x] : 0u) % kProbeSlots;
            for (int j = 1; j < 11; ++j) q4p_lds[j] = 0ull;
        }
        q4p_lds[i] = __builtin_amdgcn_s_memrealtime();
        if (i == 0) q4p_lds[11] = __builtin_amdgcn_s_memtime();
        if (i == 10) q4p_lds[12] = __builtin_amdgcn_s_memtime();
        if (i == 10 && blockIdx.x < kProbeWgs) {
            for (int j = 0; j < 16; ++j) q4p_buf[q4p_slot][blockIdx.x][j] = q4p_lds[j];
            for (int w = 0; w < 8; ++w)
                for (int j = 0; j < 4; ++j) q4p_buf[q4p_slot][blockIdx.x][16 + 4 * w + j] = q4p_wlds[w][j];
            q4p_count[blockIdx.x] += 1u;
        }
    }
}

#define Q4MOE_WAVE_MARK(i) q4p_wave(i)
#define Q4MOE_PHASE(i) q4p_mark(i)
#include "q4moe_api.hip"

// A plain streaming read of n16 16-byte pieces (non-temporal loads, grid
// stride): the rate one launch can pull from HBM.  The xor of everything
// read is stored only when `flag` is set (never by the probe), so that the
// loads stay.
__global__ __launch_bounds__(256) void k_probe_stream(const uint4* src, size_t n16, int flag, uint4* sink) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + stride));
        const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + 2 * stride));
        const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + 3 * stride));
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
    if (flag) sink[blockIdx.x * 256 + threadIdx.x] = make_uint4(acc.x, acc.y, acc.z, acc.w);
}

// An empty kernel of the one-launch decode's shape (it reads one argument
// and stores nothing unless `flag` is set, which the probe never does).
__global__ __launch_bounds__(512) void k_probe_empty(int flag, int* out) {
    if (flag && threadIdx.x == 0) out[blockIdx.x] = 1;
}

// A kernel that holds its workgroups for `ticks` of the 100 MHz clock (each
// wave spins on the clock until that much time has passed since it started:
// a wait that always ends), and records the launch's first start and last
// end (device clock) in t[2 node], t[2 node + 1].  A graph of these keeps the
// GPU busy longer than the host needs to submit it, so the gaps between the
// recorded ends and starts are the device-side cost between graph nodes.
__global__ __launch_bounds__(512) void k_probe_spin(int node, unsigned long long ticks, unsigned long long* t) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) atomicMin(&t[2 * node], t0);
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(&t[2 * node + 1], (unsigned long long)__builtin_amdgcn_s_memrealtime());
}

extern "C" {

// The phase table and the launch count.
int q4p_read(void* host, unsigned* nlaunch) {
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(q4p_buf), sizeof(q4p_buf)) != hipSuccess) return 1;
    if (hipMemcpyFromSymbol(nlaunch, HIP_SYMBOL(q4p_count), 4) != hipSuccess) return 2;  // workgroup 0's
    return 0;
}

// One streaming read of `bytes` (a multiple of 16) with `grid` workgroups.
int q4p_stream(const void* src, size_t bytes, int grid, void* sink, void* stream) {
    if (!src || !sink || bytes % 16 != 0 || grid < 1) return 1;
    hipLaunchKernelGGL(k_probe_stream, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(src), bytes / 16, 0, static_cast<uint4*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// One spin launch (graph node `node`) of `grid` x `block` threads.
int q4p_spin(int grid, int block, int node, unsigned long long ticks, void* t, void* stream) {
    if (grid < 1 || block < 1 || block > 512 || node < 0 || !t) return 1;
    hipLaunchKernelGGL(k_probe_spin, dim3(grid), dim3(block), 0, (hipStream_t)stream, node, ticks,
                       static_cast<unsigned long long*>(t));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// One empty launch of `grid` x `block` threads.
int q4p_empty(int grid, int block, void* out, void* stream) {
    if (grid < 1 || block < 1 || block > 512 || !out) return 1;
    hipLaunchKernelGGL(k_probe_empty, dim3(grid), dim3(block), 0, (hipStream_t)stream, 0, static_cast<int*>(out));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
