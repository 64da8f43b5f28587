// Align: group the (token, slot) assignments by expert, stably, and pad each
// group to a multiple of block_m (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs
// for Qwen3.5-397B", Details: sorted routing and block_m per token bucket;
// Liger-Kernel PR #1377, Testing Done: unaligned token tails).
//
// A counting sort in three phases: histogram, scan, scatter. Each wave owns a
// contiguous range of flat indices a = t*k + j and ranks each round of 64 by
// matching experts across the wave with ballots (one per bit of the expert
// id), so the output keeps ascending a inside every expert. Up to 16384 assignments run all three phases in one workgroup of
// 1024 threads (one launch); larger problems use three launches over
// 4096-index chunks. When the two GEMMs use different block sizes, the same
// pass also writes the order padded to the second block size (an element's
// place there is its place in the first layout, shifted by the difference of
// its expert's two padded offsets).
//
// The workgroups the sort leaves idle (all but one in the single-workgroup
// launch; those past the counting ones in the first of the three launches)
// prepare gemm1's activation operand meanwhile (prep.h): the MXFP4
// quantisation, the bf16 re-layout of a strided x, or the RMSNorm by rows.
#include "prep.h"

namespace moe {
namespace {

constexpr int kThreads = 512;                // multi-block kernels
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 4096;                  // indices per workgroup (multi-block)
constexpr int kWaveItems = kChunk / kWaves;   // 512
constexpr int kFusedThreads = 1024;           // single-workgroup path
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxA = 16384;

__device__ __forceinline__ int expert_of(const AlignParams& p, int a) {
    int t = (int)((unsigned)a / (unsigned)p.k);
    int j = a - t * p.k;
    const int64_t e = (int64_t)p.ids[(int64_t)t * p.is_t + (int64_t)j * p.is_j] - p.e_off;
    return (e >= 0 && e < p.E) ? (int)e : -1;
}

// Experts of a wave's indices [lo, hi), lane-strided: eid[r] is the expert
// of index lo + 64 r + lane (-1 past hi or when invalid). All loads are
// issued before any is used.
template <int R>
__device__ void wave_load(const AlignParams& p, int lo, int hi, int (&eid)[R]) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int a = lo + r * kWave + lane;
        eid[r] = a < hi ? expert_of(p, a) : -1;
    }
}

// Lanes of a wave holding the same expert as this lane, from one ballot per
// bit of the expert id (nbits bits cover 0 .. E-1); lanes with e < 0 are in
// no lane's set.
__device__ __forceinline__ uint64_t match_expert(int e, int nbits) {
    uint64_t m = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t on = __ballot(bit);
        m &= bit ? on : ~on;
    }
    return m;
}

// set bits of m below this lane
__device__ __forceinline__ int rank_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int expert_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// per-expert counts of a wave's n indices (LDS atomics)
template <int R>
__device__ void wave_count(const int (&eid)[R], int* cnt, int n) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r * kWave >= n) break;                 // the wave's n indices are done
        if (eid[r] >= 0) atomicAdd(&cnt[eid[r]], 1);
    }
}

// Scatter [lo, hi) using base[e] as the running output position of expert e.
// In each round of 64 indices an element's rank inside its expert is the
// number of lower lanes with the same expert, so the order inside an expert
// stays ascending; the highest lane of a group advances base[e] for the next
// round. off / off2: both layouts' padded offsets (second layout optional).
template <int R>
__device__ void wave_scatter(const AlignParams& p, int lo, int hi, const int (&eid)[R], int* base,
                             const int* off, const int* off2, int nbits) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int a0 = lo + r * kWave;
        if (a0 >= hi) break;
        const int e = eid[r];
        const uint64_t m = match_expert(e, nbits);
        if (e >= 0) {
            const int rank = rank_below(m);
            const int b = base[e];
            const int v = a0 + lane;
            p.sorted[b + rank] = v;
            if (p.sorted2) p.sorted2[b + rank - off[e] + off2[e]] = v;
            if ((m >> lane) == 1ull) base[e] = b + rank + 1;
        }
    }
}

// Exclusive scan of v[0..n) in place (n <= 2 * NT); returns the total.
template <int NT>
__device__ int block_exclusive_scan(int* v, int n, int* wave_tot) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int x0 = 2 * tid < n ? v[2 * tid] : 0;
    const int x1 = 2 * tid + 1 < n ? v[2 * tid + 1] : 0;
    const int s = x0 + x1;
    int inc = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) wave_tot[w] = inc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < NW; ++i) {
            const int c = wave_tot[i];
            wave_tot[i] = run;
            run += c;
        }
        wave_tot[NW] = run;
    }
    __syncthreads();
    const int excl = wave_tot[w] + inc - s;
    if (2 * tid < n) v[2 * tid] = excl;
    if (2 * tid + 1 < n) v[2 * tid + 1] = excl + x0;
    const int total = wave_tot[NW];
    __syncthreads();
    return total;
}

// Given tot[e] (assignments per expert) in LDS: the padded offsets off[e],
// block_expert and n_padded. (Every slot of sorted already holds the sentinel
// A from an earlier pass; the scatter overwrites the real ones.)
template <int NT>
__device__ void layout_experts(const AlignParams& p, int bm, int32_t* block_expert, int32_t* n_padded,
                               int32_t* expert_block, const int* tot, int* off, int* scratch) {
    const int E = p.E;
    for (int e = threadIdx.x; e < E; e += NT) off[e] = (tot[e] + bm - 1) / bm * bm;
    __syncthreads();
    const int npad = block_exclusive_scan<NT>(off, E, scratch);
    const int nblk = npad / bm;
    // block b belongs to the last expert whose offset is <= b*bm (experts
    // without tokens share their successor's offset and own no block)
    for (int b = threadIdx.x; b < nblk; b += NT) {
        const int pos = b * bm;
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        block_expert[b] = lo;
    }
    if (expert_block) {
        for (int e = threadIdx.x; e < E; e += NT) expert_block[e] = off[e] / bm;
        if (threadIdx.x == 0) expert_block[E] = nblk;
    }
    if (threadIdx.x == 0) *n_padded = npad;
}

// the sentinel A in slots [i0, i1) of both layouts, i += stride
__device__ __forceinline__ void fill_sentinels(const AlignParams& p, int i0, int stride) {
    for (int i = i0; i < p.cap; i += stride) p.sorted[i] = p.A;
    if (p.sorted2)
        for (int i = i0; i < p.cap2; i += stride) p.sorted2[i] = p.A;
}

// both layouts (the second only when asked for)
template <int NT>
__device__ void layout_both(const AlignParams& p, const int* tot, int* off, int* off2, int* scratch) {
    layout_experts<NT>(p, p.bm, p.block_expert, p.n_padded, p.expert_block, tot, off, scratch);
    if (p.sorted2)
        layout_experts<NT>(p, p.bm2, p.block_expert2, p.n_padded2, p.expert_block2, tot, off2, scratch);
}

// Whole align in one workgroup.
__device__ void align_fused_body(const AlignParams& p) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* wcnt = lds;                          // [kFusedWaves][E]
    int* tot = wcnt + kFusedWaves * E;        // [E]
    int* off = tot + E;                       // [E]
    int* off2 = off + E;                      // [E]
    int* scratch = off2 + E;                  // [kFusedWaves + 1]
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kFusedWaves * E; i += kFusedThreads) wcnt[i] = 0;
    // sentinels everywhere first (coalesced); the barriers below order them
    // before the scatter's stores
    fill_sentinels(p, threadIdx.x, kFusedThreads);
    __syncthreads();
    const int per = (p.A + kFusedWaves - 1) / kFusedWaves;
    const int lo = min(p.A, w * per), hi = min(p.A, lo + per);
    int eid[kFusedMaxA / kFusedThreads];
    wave_load(p, lo, hi, eid);
    const int nbits = expert_bits(E);
    wave_count(eid, wcnt + w * E, hi - lo);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kFusedThreads) {
        int run = 0;
        for (int v = 0; v < kFusedWaves; ++v) {
            const int c = wcnt[v * E + e];
            wcnt[v * E + e] = run;
            run += c;
        }
        tot[e] = run;
    }
    __syncthreads();
    layout_both<kFusedThreads>(p, tot, off, off2, scratch);
    for (int e = threadIdx.x; e < E; e += kFusedThreads)
        for (int v = 0; v < kFusedWaves; ++v) wcnt[v * E + e] += off[e];
    __syncthreads();
    wave_scatter(p, lo, hi, eid, wcnt + w * E, off, off2, nbits);
}

__global__ __launch_bounds__(kFusedThreads) void align_fused(AlignParams p) { align_fused_body(p); }

// Workgroup 0 aligns; workgroups 1.. prepare the activation operand
// (neither depends on the other).
template <int KIND>
__global__ __launch_bounds__(kFusedThreads) void align_fused_prep(AlignParams p, PrepParams q) {
    if (blockIdx.x == 0) {
        align_fused_body(p);
        return;
    }
    prep_block<KIND, 0, kFusedThreads>(q, (int64_t)blockIdx.x - 1);
}

// Multi-block phase 1: counts[b][e] for chunk b (b < nchunks).
__device__ void align_count_body(const AlignParams& p, int nchunks) {
    extern __shared__ int lds[];
    const int E = p.E;
    fill_sentinels(p, blockIdx.x * kThreads + threadIdx.x, nchunks * kThreads);
    for (int i = threadIdx.x; i < E; i += kThreads) lds[i] = 0;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const int lo = min(p.A, (int)blockIdx.x * kChunk + w * kWaveItems), hi = min(p.A, lo + kWaveItems);
    int eid[kWaveItems / kWave];
    wave_load(p, lo, hi, eid);
    wave_count(eid, lds, hi - lo);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) p.counts[(int64_t)blockIdx.x * E + e] = lds[e];
}

__global__ __launch_bounds__(kThreads) void align_count(AlignParams p) { align_count_body(p, gridDim.x); }

// Workgroups past the nchunks counting ones prepare the activation operand.
template <int KIND>
__global__ __launch_bounds__(kThreads) void align_count_prep(AlignParams p, PrepParams q, int nchunks) {
    if ((int)blockIdx.x < nchunks) {
        align_count_body(p, nchunks);
        return;
    }
    prep_block<KIND, 0, kThreads>(q, (int64_t)blockIdx.x - nchunks);
}

// The row-layout RMSNorm (and the quantisation of the normalised rows) on
// its own: four rows per workgroup.
template <int NCL>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams q) {
    prep_block<kPrepNormRows, NCL, 256>(q, blockIdx.x);
}

// Multi-block phase 2: per-expert prefix over chunks, padded offsets.
__global__ __launch_bounds__(kThreads) void align_scan(AlignParams p, int nchunks) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* tot = lds;
    int* off = tot + E;
    int* off2 = off + E;
    int* scratch = off2 + E;
    // counts of one expert are read 16 chunks at a time, all loads in flight
    constexpr int kBatch = 16;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int run = 0;
        for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) c[i] = b0 + i < nchunks ? p.counts[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (b0 + i < nchunks) p.counts[(int64_t)(b0 + i) * E + e] = run;
                run += c[i];
            }
        }
        tot[e] = run;
    }
    __syncthreads();
    layout_both<kThreads>(p, tot, off, off2, scratch);
    // both layouts' offsets for the scatter, after the chunk counts
    int32_t* offs = p.counts + (int64_t)nchunks * E;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        offs[e] = off[e];
        offs[E + e] = p.sorted2 ? off2[e] : 0;
    }
    for (int e = threadIdx.x; e < E; e += kThreads)
        for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) c[i] = b0 + i < nchunks ? p.counts[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (b0 + i < nchunks) p.counts[(int64_t)(b0 + i) * E + e] = c[i] + off[e];
        }
}

// Multi-block phase 3: stable scatter of chunk b.
__global__ __launch_bounds__(kThreads) void align_scatter(AlignParams p, int nchunks) {
    extern __shared__ int lds[];
    const int E = p.E;
    int* wcnt = lds;                  // [kWaves][E]
    int* off = wcnt + kWaves * E;     // [E]
    int* off2 = off + E;              // [E]
    for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
    const int32_t* offs = p.counts + (int64_t)nchunks * E;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        off[e] = offs[e];
        off2[e] = offs[E + e];
    }
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const int lo = min(p.A, (int)blockIdx.x * kChunk + w * kWaveItems), hi = min(p.A, lo + kWaveItems);
    int eid[kWaveItems / kWave];
    wave_load(p, lo, hi, eid);
    const int nbits = expert_bits(E);
    wave_count(eid, wcnt + w * E, hi - lo);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int run = p.counts[(int64_t)blockIdx.x * E + e];
        for (int v = 0; v < kWaves; ++v) {
            const int c = wcnt[v * E + e];
            wcnt[v * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    wave_scatter(p, lo, hi, eid, wcnt + w * E, off, off2, nbits);
}

bool use_fused(int A, int E) {
    return A <= kFusedMaxA && (size_t)(kFusedWaves + 3) * E * sizeof(int) + 256 <= 64 * 1024;
}

}  // namespace

size_t align_scratch_bytes(int64_t A, int32_t E) {
    if (use_fused((int)A, E)) return 0;
    const int64_t nchunks = (A + kChunk - 1) / kChunk;
    return (size_t)(nchunks + 2) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_align_prep(const AlignParams& p, int kind, const PrepParams& q, hipStream_t s) {
    const int E = p.E;
    if (use_fused(p.A, E)) {
        const size_t lds = sizeof(int) * ((size_t)kFusedWaves * E + 3 * E + kFusedWaves + 1);
        const dim3 grid((unsigned)(1 + prep_blocks(kind, q, kFusedThreads)));
        switch (kind) {
        case 0: hipLaunchKernelGGL(align_fused, dim3(1), dim3(kFusedThreads), lds, s, p); break;
        case kPrepQuant: hipLaunchKernelGGL(align_fused_prep<kPrepQuant>, grid, dim3(kFusedThreads), lds, s, p, q); break;
        case kPrepPack: hipLaunchKernelGGL(align_fused_prep<kPrepPack>, grid, dim3(kFusedThreads), lds, s, p, q); break;
        case kPrepNormRows:
            hipLaunchKernelGGL(align_fused_prep<kPrepNormRows>, grid, dim3(kFusedThreads), lds, s, p, q);
            break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const int nchunks = (p.A + kChunk - 1) / kChunk;
    const size_t lds_c = sizeof(int) * (size_t)E;
    const dim3 grid((unsigned)(nchunks + prep_blocks(kind, q, kThreads)));
    switch (kind) {
    case 0: hipLaunchKernelGGL(align_count, dim3(nchunks), dim3(kThreads), lds_c, s, p); break;
    case kPrepQuant: hipLaunchKernelGGL(align_count_prep<kPrepQuant>, grid, dim3(kThreads), lds_c, s, p, q, nchunks); break;
    case kPrepPack: hipLaunchKernelGGL(align_count_prep<kPrepPack>, grid, dim3(kThreads), lds_c, s, p, q, nchunks); break;
    case kPrepNormRows:
        hipLaunchKernelGGL(align_count_prep<kPrepNormRows>, grid, dim3(kThreads), lds_c, s, p, q, nchunks);
        break;
    default: return hipErrorInvalidValue;
    }
    const size_t lds_s = sizeof(int) * (3 * (size_t)E + kWaves + 1);
    hipLaunchKernelGGL(align_scan, dim3(1), dim3(kThreads), lds_s, s, p, nchunks);
    const size_t lds_x = sizeof(int) * ((size_t)kWaves + 2) * E;
    hipLaunchKernelGGL(align_scatter, dim3(nchunks), dim3(kThreads), lds_x, s, p, nchunks);
    return hipGetLastError();
}

hipError_t launch_align(const AlignParams& p, hipStream_t s) { return launch_align_prep(p, 0, PrepParams{}, s); }

hipError_t launch_prep_norm_rows(const PrepParams& q, hipStream_t s) {
    if (q.n.T == 0) return hipSuccess;
    const dim3 grid((unsigned)prep_blocks(kPrepNormRows, q, 256));
    if (q.n.H <= 512 * 8)
        hipLaunchKernelGGL(prep_kernel<8>, grid, dim3(256), 0, s, q);
    else if (q.n.H <= 512 * 16)
        hipLaunchKernelGGL(prep_kernel<16>, grid, dim3(256), 0, s, q);
    else
        hipLaunchKernelGGL(prep_kernel<0>, grid, dim3(256), 0, s, q);
    return hipGetLastError();
}

}  // namespace moe
