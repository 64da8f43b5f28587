// RMSNorm of the activation rows ahead of gemm1:
//   out[t, h] = bf16( (x[t, h] * r_t) * w[h] ),  r_t = 1 / sqrt(ss_t / H + eps),
// ss_t the fp32 sum of x[t, h]^2 over the row (LightLLM issue #1467, Summary
// and Expected Behavior: the variance and the normalize pass both read the
// row through its last-dim stride; the issue's reference multiplies the
// normalised row by the weight).
//
// The sum has one fixed order for every layout, so a transposed activation
// gives the same bits as a contiguous one: chunk c holds elements 8c .. 8c+7;
// partial q (q = 0..63) is an fmaf chain over the chunks c = q, q + 64, ...
// in ascending order, element by element; the 64 partials are then added as a
// wave64 xor butterfly (distance 32, 16, ..., 1).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float norm_weight(const NormParams& p, int64_t h) {
    return norm_weight_at(p.w, p.w_f32 != 0, p.ws, h);
}

// The 8 values of chunk c of row xr.
__device__ __forceinline__ void load_chunk(const uint16_t* xr, int64_t s_h, bool vec, int64_t c, float (&v)[8]) {
    if (vec) {
        const uint4 q = *reinterpret_cast<const uint4*>(xr + 8 * c);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(xr[(8 * c + i) * s_h]);
    }
}

// The 8 weights of chunk c (one or two 16-byte loads when w is contiguous
// and aligned).
__device__ __forceinline__ void load_weights(const NormParams& p, bool wvec, int64_t c, float (&wv)[8]) {
    if (wvec && p.w_f32) {
        const float4* w4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.w) + 8 * c);
        const float4 a = w4[0], b = w4[1];
        wv[0] = a.x; wv[1] = a.y; wv[2] = a.z; wv[3] = a.w;
        wv[4] = b.x; wv[5] = b.y; wv[6] = b.z; wv[7] = b.w;
    } else if (wvec) {
        const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.w) + 8 * c);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wv[2 * i] = __uint_as_float(u[i] << 16);
            wv[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = norm_weight(p, 8 * c + i);
    }
}

__device__ __forceinline__ bool weights_vec(const NormParams& p) {
    return p.ws == 1 && (((uintptr_t)p.w) & 15u) == 0;
}

// Normalised chunk c of a row to the output row dr (element stride os_h).
__device__ __forceinline__ void store_chunk(const NormParams& p, const float (&v)[8], const float (&wv)[8],
                                            float r, int64_t c, uint16_t* dr) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = f32_to_bf16_bits((v[i] * r) * wv[i]);
    uint16_t* d = dr + 8 * c * p.os_h;
    if (p.os_h == 1 && (((uintptr_t)d) & 15u) == 0) {
        *reinterpret_cast<uint4*>(d) =
            make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i * p.os_h] = (uint16_t)b[i];
    }
}

// Rows with unit last-dim stride: one wave per row, lane q owns partial q.
// With NCL > 0 (H <= 512 NCL) a lane loads all its chunks and their weights
// at once and keeps them in registers for the second pass; NCL = 0 loops.
template <int NCL>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(NormParams p) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.T) return;
    const int q = threadIdx.x & 63;
    const uint16_t* xr = p.x + t * p.xs_t;
    const bool vec = (((uintptr_t)xr) & 15u) == 0;
    const int64_t nc = p.H / 8;
    uint16_t* dr = p.out + t * p.os_t;
    float acc = 0.f;
    const bool wvec = weights_vec(p);
    if constexpr (NCL > 0) {
        // every load of the row before any store: stores share the load
        // counter, and a wait for a later load would also wait for them
        float v[NCL][8], wv[NCL][8];
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int64_t c = q + 64 * j;
            if (c < nc) {
                load_chunk(xr, 1, vec, c, v[j]);
                load_weights(p, wvec, c, wv[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            if (q + 64 * j < nc) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[j][i], v[j][i], acc);
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
        const float r = rms_scale(acc, p.H, p.eps);
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int64_t c = q + 64 * j;
            if (c < nc) store_chunk(p, v[j], wv[j], r, c, dr);
        }
    } else {
        for (int64_t c = q; c < nc; c += 64) {
            float v[8];
            load_chunk(xr, 1, vec, c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[i], v[i], acc);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
        const float r = rms_scale(acc, p.H, p.eps);
        for (int64_t c = q; c < nc; c += 64) {
            float v[8], wv[8];
            load_chunk(xr, 1, vec, c, v);
            load_weights(p, wvec, c, wv);
            store_chunk(p, v, wv, r, c, dr);
        }
    }
}

// Any strides: 64 rows per workgroup, lane = row (an activation stored
// transposed, s_t = 1, is read with unit stride across the lanes). Wave w of
// 16 computes partials q = w, w + 16, w + 32, w + 48 of every row, each with
// the 8 chunks c = q + 64 j of a group loaded at once; the partials meet in
// LDS and wave 0 adds them in the butterfly's pairing; then the 16 waves
// normalise chunks c = 16 y + w + 16 S j (y = blockIdx.y of S column slices;
// S > 1 spreads the stores of few rows over more CUs, each slice
// recomputing the sums), loading 4 chunks before storing them.
__global__ __launch_bounds__(1024) void rmsnorm_cols_kernel(NormParams p) {
    __shared__ float part[64][65];
    __shared__ float scale[64];
    // the wave index as a uniform value keeps chunk offsets in scalar registers
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * 64 + lane;
    const bool live = t < p.T;
    const uint16_t* xr = p.x + (live ? t : 0) * p.xs_t;
    const int64_t nc = p.H / 8;
#pragma unroll 1
    for (int qi = 0; qi < 4; ++qi) {
        const int q = w + 16 * qi;
        float acc = 0.f;
#pragma unroll 1
        for (int64_t c0 = q; c0 < nc; c0 += 64 * 8) {
            float v[8][8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + 64 * j < nc) load_chunk(xr, p.xs_h, false, c0 + 64 * j, v[j]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + 64 * j < nc) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[j][i], v[j][i], acc);
                }
            }
        }
        part[q][lane] = acc;
    }
    __syncthreads();
    if (w == 0) {
        float v[64];
#pragma unroll
        for (int q = 0; q < 64; ++q) v[q] = part[q][lane];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int q = 0; q < m; ++q) v[q] = v[q] + v[q + m];
        }
        scale[lane] = rms_scale(v[0], p.H, p.eps);
    }
    __syncthreads();
    if (!live) return;
    const float r = scale[lane];
    uint16_t* dr = p.out + t * p.os_t;
    const bool wvec = weights_vec(p);
    const int64_t step = 16 * (int64_t)gridDim.y;
#pragma unroll 1
    for (int64_t c0 = 16 * (int64_t)blockIdx.y + w; c0 < nc; c0 += 4 * step) {
        float v[4][8], wv[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = c0 + step * j;
            if (c < nc) {
                load_chunk(xr, p.xs_h, false, c, v[j]);
                load_weights(p, wvec, c, wv[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = c0 + step * j;
            if (c < nc) store_chunk(p, v[j], wv[j], r, c, dr);
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    const dim3 rows((unsigned)((p.T + 3) / 4));
    if (p.xs_h != 1) {
        const int64_t blocks = (p.T + 63) / 64;
        int slices = 1;
        while (slices < 16 && blocks * slices * 2 <= 256 && p.H / 8 >= 16 * slices * 2) slices *= 2;
        hipLaunchKernelGGL(rmsnorm_cols_kernel, dim3((unsigned)blocks, (unsigned)slices), dim3(1024), 0, s, p);
    }
    else if (p.H <= 512 * 8)
        hipLaunchKernelGGL(rmsnorm_rows_kernel<8>, rows, dim3(256), 0, s, p);
    else if (p.H <= 512 * 16)
        hipLaunchKernelGGL(rmsnorm_rows_kernel<16>, rows, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(rmsnorm_rows_kernel<0>, rows, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
