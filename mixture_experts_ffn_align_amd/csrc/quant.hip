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

// dst[t, h] = src[t*s_t + h*s_h] for an activation whose rows are not
// 16-byte runs (last-dim stride != 1, or unaligned rows). A workgroup moves a
// 64-token x 64-column tile through LDS: lanes walk t on the read side, so an
// activation stored transposed (s_t = 1) is read in 128-byte runs, and eight
// lanes write each destination row's 128 bytes on the store side, so every
// store fills whole cache lines.
constexpr int kPackTile = 64;
__global__ __launch_bounds__(256) void pack_bf16_kernel(PackParams p) {
    __shared__ uint16_t tile[kPackTile][kPackTile + 8];
    const int64_t t0 = (int64_t)blockIdx.x * kPackTile, h0 = (int64_t)blockIdx.y * kPackTile;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll 4
    for (int i = 0; i < kPackTile / 4; ++i) {
        const int hl = i * 4 + wv;
        const int64_t t = t0 + lane, h = h0 + hl;
        if (t < p.T && h < p.H) tile[lane][hl] = p.src[t * p.s_t + h * p.s_h];
    }
    __syncthreads();
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int tl = (threadIdx.x >> 3) + 32 * pass;
        const int64_t t = t0 + tl, h = h0 + chunk * 8;
        if (t < p.T && h < p.H) {
            const uint16_t* r = &tile[tl][chunk * 8];
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (uint32_t)r[2 * i] | ((uint32_t)r[2 * i + 1] << 16);
            *reinterpret_cast<uint4*>(p.dst + t * p.H + h) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
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
    dim3 grid((unsigned)((p.T + kPackTile - 1) / kPackTile), (unsigned)((p.H + kPackTile - 1) / kPackTile));
    hipLaunchKernelGGL(pack_bf16_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
