// bf16 -> MXFP4: e2m1 codes with one e8m0 scale per 32 elements along K
// (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for Qwen3.5-397B", Details:
// float4_e2m1fn_x2 weights and activations, QuantType.per_1x32). Also the
// bf16 re-layout of an activation whose last-dim stride is not 1 (LightLLM
// issue #1467: such inputs must be read through their stride, not as if
// contiguous).
#include "prep.h"

namespace moe {
namespace {

// One thread per group of 32 values.
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(QuantParams p) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < p.E * p.R * (p.K / 32)) quant_group_mxfp4(p, g);
}

// dst[t, h] = src[t*s_t + h*s_h] for an activation whose rows are not
// 16-byte runs (last-dim stride != 1, or unaligned rows): one 64 x 64 tile
// per workgroup through LDS (the tile body is shared with the align launch).
__global__ __launch_bounds__(256) void pack_bf16_kernel(PackParams p) {
    __shared__ PackTileLds tile;
    const int64_t t0 = (int64_t)blockIdx.x * kPackTile, h0 = (int64_t)blockIdx.y * kPackTile;
    prep_pack_load(p, t0, h0, threadIdx.x, tile);
    __syncthreads();
    prep_pack_store(p, t0, h0, threadIdx.x, tile);
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
