// Combine: out[t, n] = bf16(sum over slots j = 0..k-1 of w[t, j] * y[t, j, n]),
// y stored in bf16 and widened exactly to fp32, accumulated with fmaf in slot
// order from +0 and rounded once. Slots whose id lies outside
// [e_off, e_off + E) contribute nothing and their rows are not read. No
// atomics, so the result is the same on every run and for every input layout.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

// Each thread produces CP (4 or 8) consecutive columns of one token: one 8- or
// 16-byte load of y per slot. Slots go in groups of G (8, or 16 for more
// than 8 slots, so that 10 or 11 slots are one group and every y load of
// the thread is in flight before the first wait).
template <int CP, int G>
__device__ __forceinline__ void combine_one(const CombineParams& p, int64_t t, int q) {
    const int n = q * CP;
    float acc[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) acc[i] = 0.f;
    // slots in groups of G: the group's ids and weights (the same for the
    // whole workgroup), then its y loads, then the fmaf chain in slot order,
    // so that a few tokens wait on one load latency per group, not per slot
    for (int j0 = 0; j0 < p.k; j0 += G) {
        int32_t id[G];
        float wt[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = min(j0 + jj, p.k - 1);     // past k: re-read the last slot, dropped below
            id[jj] = p.ids[(int64_t)t * p.is_t + (int64_t)j * p.is_j];
            wt[jj] = p.w[(int64_t)t * p.ws_t + (int64_t)j * p.ws_j];
        }
        __builtin_amdgcn_sched_barrier(0);
        bool live[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int64_t e = (int64_t)__builtin_amdgcn_readfirstlane(id[jj]) - p.e_off;
            live[jj] = j0 + jj < p.k && e >= 0 && e < p.E;
        }
        uint32_t u[G][CP / 2];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            if (!live[jj]) continue;
            const uint16_t* src = p.y + (int64_t)t * p.ys_t + (int64_t)(j0 + jj) * p.ys_j + n;
            if constexpr (CP == 8) {
                const uint4 v = *reinterpret_cast<const uint4*>(src);
                u[jj][0] = v.x; u[jj][1] = v.y; u[jj][2] = v.z; u[jj][3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(src);
                u[jj][0] = v.x; u[jj][1] = v.y;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            if (!live[jj]) continue;
#pragma unroll
            for (int i = 0; i < CP / 2; ++i) {
                acc[2 * i] = __builtin_fmaf(wt[jj], __uint_as_float(u[jj][i] << 16), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(wt[jj], __uint_as_float(u[jj][i] & 0xffff0000u), acc[2 * i + 1]);
            }
        }
    }
    uint16_t* o = p.out + (int64_t)t * p.os_t;
    uint32_t b[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) b[i] = f32_to_bf16_bits(acc[i]);
    if (p.os_h == 1 && (((uintptr_t)(o + n)) & (2 * CP - 1)) == 0) {
        if constexpr (CP == 8)
            *reinterpret_cast<uint4*>(o + n) =
                make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
        else
            *reinterpret_cast<uint2*>(o + n) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    } else {
#pragma unroll
        for (int i = 0; i < CP; ++i) o[(int64_t)(n + i) * p.os_h] = (uint16_t)b[i];
    }
}

// Workgroup b covers token b / nqb, column group b % nqb; the grid is capped
// and strides over the (token, column group) pairs.
template <int CP, int G>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const int ncol = p.H / CP;
    const int nqb = (ncol + 255) / 256;               // workgroups per token
    const int64_t total = (int64_t)p.T * nqb;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t t = b / nqb;
        const int q = (int)(b % nqb) * 256 + threadIdx.x;
        if (q < ncol) combine_one<CP, G>(p, t, q);
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    const int cp = p.H % 8 == 0 ? 8 : 4;
    const int64_t ncol = p.H / cp;
    const int64_t blocks = ((ncol + 255) / 256) * (int64_t)p.T;
    dim3 grid((unsigned)std::min<int64_t>(blocks, (int64_t)1 << 22));
    const bool g16 = p.k > 8;
    if (cp == 8 && g16) hipLaunchKernelGGL((combine_kernel<8, 16>), grid, dim3(256), 0, s, p);
    else if (cp == 8) hipLaunchKernelGGL((combine_kernel<8, 8>), grid, dim3(256), 0, s, p);
    else if (g16) hipLaunchKernelGGL((combine_kernel<4, 16>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<4, 8>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
