// Combine: out[t, n] = bf16(sum over slots j = 0..k-1 of w[t, j] * y[t*k + j, n]),
// y read as fp32 (bf16 mode) or as bf16 widened exactly to fp32 (MXFP4 mode),
// accumulated with fmaf in slot order from +0 and rounded once. Slots whose
// id lies outside [0, E) contribute nothing. No atomics, so the result is the
// same on every run and for every input layout.
#include "moe_internal.h"

namespace moe {
namespace {

// Each thread produces 4 consecutive columns of one token; y is fp32 or bf16.
template <bool Y16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const int nqb = (p.H / 4 + 255) / 256;            // workgroups per token
    const int t = blockIdx.x / nqb;
    const int q = (blockIdx.x % nqb) * 256 + threadIdx.x;   // column quad within the token
    const int n = q * 4;
    if (n >= p.H) return;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.k; ++j) {
        const int e = p.ids[(int64_t)t * p.is_t + (int64_t)j * p.is_j];
        if (e < 0 || e >= p.E) continue;
        const float wt = p.w[(int64_t)t * p.ws_t + (int64_t)j * p.ws_j];
        const int64_t off = ((int64_t)t * p.k + j) * p.H + n;
        f32x4_t v;
        if constexpr (Y16) {
            const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.y) + off);
            v = f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                        __uint_as_float(u.y & 0xffff0000u)};
        } else {
            v = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(p.y) + off);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(wt, v[i], acc[i]);
    }
    uint16_t* o = p.out + (int64_t)t * p.os_t;
    const uint32_t b0 = f32_to_bf16_bits(acc[0]), b1 = f32_to_bf16_bits(acc[1]);
    const uint32_t b2 = f32_to_bf16_bits(acc[2]), b3 = f32_to_bf16_bits(acc[3]);
    if (p.os_h == 1 && (((uintptr_t)(o + n)) & 7u) == 0) {
        *reinterpret_cast<uint2*>(o + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else {
        o[(int64_t)(n + 0) * p.os_h] = (uint16_t)b0;
        o[(int64_t)(n + 1) * p.os_h] = (uint16_t)b1;
        o[(int64_t)(n + 2) * p.os_h] = (uint16_t)b2;
        o[(int64_t)(n + 3) * p.os_h] = (uint16_t)b3;
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    const int quads = p.H / 4;
    dim3 grid((unsigned)(((quads + 255) / 256) * (int64_t)p.T));
    if (p.y_bf16) hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
