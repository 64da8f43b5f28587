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
#include "prep.h"

namespace moe {
namespace {

// Rows with unit last-dim stride: one wave per row (four per workgroup).
template <int NCL>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(NormParams p) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.T) return;
    prep_norm_row<NCL>(p, t, threadIdx.x & 63);
}

// Any strides: 64 rows per workgroup of 16 waves, blockIdx.y one of
// gridDim.y column slices of the stores.
__global__ __launch_bounds__(1024) void rmsnorm_cols_kernel(NormParams p) {
    __shared__ PrepNormColsLds L;
    prep_norm_cols<16>(p, blockIdx.x, blockIdx.y, gridDim.y, L);
}

}  // namespace

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    const dim3 rows((unsigned)((p.T + 3) / 4));
    if (p.xs_h != 1 && p.os_h == 1 && p.os_t == p.H && (((uintptr_t)p.out) & 15u) == 0 && p.H <= 512 * 16) {
        // A strided x into a contiguous out: re-lay x into out (64 x 64
        // tiles through LDS, coalesced on both sides), then normalise out in
        // place by rows, each wave holding its whole row in registers before
        // it stores (NCL > 0). Same order, same bits as the column kernel,
        // which leaves few workgroups each reading 64 whole rows.
        PackParams pk{};
        pk.src = p.x;
        pk.s_t = p.xs_t;
        pk.s_h = p.xs_h;
        pk.dst = p.out;
        pk.T = p.T;
        pk.H = p.H;
        hipError_t e = launch_pack_bf16(pk, s);
        if (e != hipSuccess) return e;
        NormParams q = p;
        q.x = p.out;
        q.xs_t = p.H;
        q.xs_h = 1;
        if (p.H <= 512 * 8)
            hipLaunchKernelGGL(rmsnorm_rows_kernel<8>, rows, dim3(256), 0, s, q);
        else
            hipLaunchKernelGGL(rmsnorm_rows_kernel<16>, rows, dim3(256), 0, s, q);
        return hipGetLastError();
    }
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
