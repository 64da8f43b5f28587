// bf16 -> MXFP4: e2m1 codes with one e8m0 scale per 32 elements along K
// (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for Qwen3.5-397B", Details:
// float4_e2m1fn_x2 weights and activations, QuantType.per_1x32). Also the
// bf16 re-layout of an activation whose last-dim stride is not 1 (LightLLM
// issue #1467: such inputs must be read through their stride, not as if
// contiguous).
#include "moe_internal.h"

namespace moe {
namespace {

// One thread per group of 32 values.
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(QuantParams p) {
    const int64_t groups_per_row = p.K / 32;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = p.E * p.R * groups_per_row;
    if (g >= total) return;
    const int64_t kb = g % groups_per_row;
    const int64_t rr = g / groups_per_row;
    const int64_t r = rr % p.R;
    const int64_t e = rr / p.R;
    const uint16_t* src = p.src + e * p.ss_e + r * p.ss_r + kb * 32 * p.ss_k;
    uint16_t v[32];
    const bool vec = p.ss_k == 1 && ((uintptr_t)src & 15u) == 0;
    if (vec) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 q = s4[i];
            uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[i * 8 + 2 * h] = (uint16_t)(w[h] & 0xffffu);
                v[i * 8 + 2 * h + 1] = (uint16_t)(w[h] >> 16);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = src[(int64_t)i * p.ss_k];
    }
    // |v| compares as an integer for finite bf16 values
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        uint32_t a = v[i] & 0x7fffu;
        amax = a > amax ? a : amax;
    }
    const int s = group_exponent(amax << 16);
    const E2m1Thresholds th = e2m1_thresholds(s);
    uint32_t packed[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code((uint32_t)v[q * 8 + i] << 16, th) << (4 * i);
        packed[q] = word;
    }
    uint8_t* dst = p.codes + e * p.cs_e + r * p.cs_r + kb * 16;
    if (((uintptr_t)dst & 15u) == 0) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[i] = (uint8_t)(packed[i / 4] >> (8 * (i % 4)));
    }
    p.scales[e * p.xs_e + r * p.xs_r + kb] = (uint8_t)(s + 127);
}

// dst[t, h] = src[t*s_t + h*s_h]; 8 columns per thread, lanes walk t so that
// an activation stored transposed (s_t = 1) is read with unit stride.
__global__ __launch_bounds__(256) void pack_bf16_kernel(PackParams p) {
    const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const int64_t h0 = ((int64_t)blockIdx.y * 4 + (threadIdx.x >> 6)) * 8;
    if (t >= p.T || h0 >= p.H) return;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = p.src[t * p.s_t + (h0 + 2 * i) * p.s_h];
        uint32_t hi = p.src[t * p.s_t + (h0 + 2 * i + 1) * p.s_h];
        w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(p.dst + t * p.H + h0) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

hipError_t launch_quant_mxfp4(const QuantParams& p, hipStream_t s) {
    const int64_t total = p.E * p.R * (p.K / 32);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(const PackParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    dim3 grid((unsigned)((p.T + 63) / 64), (unsigned)((p.H / 8 + 3) / 4));
    hipLaunchKernelGGL(pack_bf16_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
