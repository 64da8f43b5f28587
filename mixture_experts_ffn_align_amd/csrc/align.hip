// Align: group the (token, slot) assignments by expert, stably, and pad each
// group to a multiple of block_m (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs
// for Qwen3.5-397B", Details: sorted routing and block_m per token bucket;
// Liger-Kernel PR #1377, Testing Done: unaligned token tails).
//
// A counting sort in three phases: histogram, scan, scatter. Each wave owns a
// contiguous range of flat indices a = t*k + j; within a wave, lanes with the
// same expert are ranked by a ballot over lower lanes, so the output keeps
// ascending a inside every expert. Small problems run all three phases in one
// workgroup (one launch); larger ones use three launches over 16384-index
// chunks.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 16384;                 // indices per workgroup (multi-block)
constexpr int kWaveItems = kChunk / kWaves;   // 2048

__device__ __forceinline__ int expert_of(const AlignParams& p, int a) {
    int t = (int)((unsigned)a / (unsigned)p.k);
    int j = a - t * p.k;
    int e = p.ids[(int64_t)t * p.is_t + (int64_t)j * p.is_j];
    return (e >= 0 && e < p.E) ? e : -1;
}

__device__ void wave_count(const AlignParams& p, int lo, int hi, int* cnt) {
    for (int a = lo + lane_id(); a < hi; a += kWave) {
        int e = expert_of(p, a);
        if (e >= 0) atomicAdd(&cnt[e], 1);
    }
}

// Scatter [lo, hi) using base[e] as the running output position of expert e.
__device__ void wave_scatter(const AlignParams& p, int lo, int hi, int* base) {
    const int lane = lane_id();
    for (int a0 = lo; a0 < hi; a0 += kWave) {
        const int a = a0 + lane;
        int e = a < hi ? expert_of(p, a) : -1;
        const bool valid = e >= 0;
        uint64_t active = __ballot(valid);
        while (active) {
            const int leader = __ffsll((unsigned long long)active) - 1;
            const int e0 = __shfl(e, leader);
            const uint64_t m = __ballot(valid && e == e0);
            const int b = base[e0];
            if (valid && e == e0) p.sorted[b + __popcll(m & lanemask_lt())] = a;
            if (lane == leader) base[e0] = b + __popcll(m);
            active &= ~m;
        }
    }
}

// Exclusive scan of v[0..n) in place (n <= 2 * kThreads); returns the total.
__device__ int block_exclusive_scan(int* v, int n, int* wave_tot) {
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    // two items per thread: [2*tid, 2*tid+1]
    int x0 = 2 * tid < n ? v[2 * tid] : 0;
    int x1 = 2 * tid + 1 < n ? v[2 * tid + 1] : 0;
    int s = x0 + x1;
    int inc = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) wave_tot[w] = inc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < kWaves; ++i) {
            int c = wave_tot[i];
            wave_tot[i] = run;
            run += c;
        }
        wave_tot[kWaves] = run;
    }
    __syncthreads();
    int excl = wave_tot[w] + inc - s;
    if (2 * tid < n) v[2 * tid] = excl;
    if (2 * tid + 1 < n) v[2 * tid + 1] = excl + x0;
    int total = wave_tot[kWaves];
    __syncthreads();
    return total;
}

// Given tot[e] (assignments per expert) in LDS: compute the padded offsets
// off[e], write block_expert and the sentinels, and n_padded.
__device__ void layout_experts(const AlignParams& p, const int* tot, int* off, int* scratch) {
    const int E = p.E, bm = p.bm;
    for (int e = threadIdx.x; e < E; e += kThreads) off[e] = (tot[e] + bm - 1) / bm * bm;
    __syncthreads();
    const int npad = block_exclusive_scan(off, E, scratch);
    const int nblk = npad / bm;
    // block b belongs to the last expert whose offset is <= b*bm
    for (int b = threadIdx.x; b < nblk; b += kThreads) {
        const int pos = b * bm;
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        // skip experts with no blocks that share the same offset
        const int e = lo;
        p.block_expert[b] = e;
        const int fill_from = off[e] + tot[e];
        const int end = pos + bm;
        for (int q = (fill_from > pos ? fill_from : pos); q < end; ++q) p.sorted[q] = p.A;
    }
    if (threadIdx.x == 0) *p.n_padded = npad;
}

// Whole align in one workgroup.
__global__ __launch_bounds__(kThreads) void align_fused(AlignParams p) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* wcnt = lds;                     // [kWaves][E]
    int* tot = wcnt + kWaves * E;        // [E]
    int* off = tot + E;                  // [E]
    int* scratch = off + E;              // [kWaves + 1]
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();
    const int per = (p.A + kWaves - 1) / kWaves;
    const int lo = min(p.A, w * per), hi = min(p.A, lo + per);
    wave_count(p, lo, hi, wcnt + w * E);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int run = 0;
        for (int v = 0; v < kWaves; ++v) {
            int c = wcnt[v * E + e];
            wcnt[v * E + e] = run;
            run += c;
        }
        tot[e] = run;
    }
    __syncthreads();
    layout_experts(p, tot, off, scratch);
    for (int e = threadIdx.x; e < E; e += kThreads)
        for (int v = 0; v < kWaves; ++v) wcnt[v * E + e] += off[e];
    __syncthreads();
    wave_scatter(p, lo, hi, wcnt + w * E);
}

// Multi-block phase 1: counts[b][e] for chunk b.
__global__ __launch_bounds__(kThreads) void align_count(AlignParams p) {
    extern __shared__ int lds[];
    const int E = p.E;
    for (int i = threadIdx.x; i < E; i += kThreads) lds[i] = 0;
    __syncthreads();
    const int base = blockIdx.x * kChunk;
    const int w = threadIdx.x >> 6;
    const int lo = min(p.A, base + w * kWaveItems), hi = min(p.A, lo + kWaveItems);
    wave_count(p, lo, hi, lds);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) p.counts[(int64_t)blockIdx.x * E + e] = lds[e];
}

// Multi-block phase 2: per-expert prefix over chunks, padded offsets.
__global__ __launch_bounds__(kThreads) void align_scan(AlignParams p, int nchunks) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* tot = lds;
    int* off = tot + E;
    int* scratch = off + E;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int run = 0;
        for (int b = 0; b < nchunks; ++b) {
            int c = p.counts[(int64_t)b * E + e];
            p.counts[(int64_t)b * E + e] = run;
            run += c;
        }
        tot[e] = run;
    }
    __syncthreads();
    layout_experts(p, tot, off, scratch);
    for (int e = threadIdx.x; e < E; e += kThreads)
        for (int b = 0; b < nchunks; ++b) p.counts[(int64_t)b * E + e] += off[e];
}

// Multi-block phase 3: stable scatter of chunk b.
__global__ __launch_bounds__(kThreads) void align_scatter(AlignParams p) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* wcnt = lds;   // [kWaves][E]
    for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();
    const int base = blockIdx.x * kChunk;
    const int w = threadIdx.x >> 6;
    const int lo = min(p.A, base + w * kWaveItems), hi = min(p.A, lo + kWaveItems);
    wave_count(p, lo, hi, wcnt + w * E);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int run = p.counts[(int64_t)blockIdx.x * E + e];
        for (int v = 0; v < kWaves; ++v) {
            int c = wcnt[v * E + e];
            wcnt[v * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    wave_scatter(p, lo, hi, wcnt + w * E);
}

}  // namespace

size_t align_scratch_bytes(int64_t A, int32_t E) {
    int64_t nchunks = (A + kChunk - 1) / kChunk;
    return (size_t)(nchunks > 1 ? nchunks : 0) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_align(const AlignParams& p, hipStream_t s) {
    const int E = p.E;
    const int nchunks = (p.A + kChunk - 1) / kChunk;
    if (nchunks <= 1) {
        size_t lds = sizeof(int) * ((size_t)kWaves * E + 2 * E + kWaves + 1);
        hipLaunchKernelGGL(align_fused, dim3(1), dim3(kThreads), lds, s, p);
        return hipGetLastError();
    }
    size_t lds_c = sizeof(int) * (size_t)E;
    hipLaunchKernelGGL(align_count, dim3(nchunks), dim3(kThreads), lds_c, s, p);
    size_t lds_s = sizeof(int) * (2 * (size_t)E + kWaves + 1);
    hipLaunchKernelGGL(align_scan, dim3(1), dim3(kThreads), lds_s, s, p, nchunks);
    size_t lds_x = sizeof(int) * (size_t)kWaves * E;
    hipLaunchKernelGGL(align_scatter, dim3(nchunks), dim3(kThreads), lds_x, s, p);
    return hipGetLastError();
}

}  // namespace moe
