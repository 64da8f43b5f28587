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
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < p.E * p.R * (p.K / 32)) quant_group_mxfp4(p, g);
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
