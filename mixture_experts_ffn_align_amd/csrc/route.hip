// Router: top-k over the softmax of the router logits, renormalised
// (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for Qwen3.5-397B", Summary:
// 512/10 unfused routing and 513/11 with a shared expert fused in).
//
// One wavefront per token. Softmax is monotone, so the k largest
// probabilities are the k largest logits: each lane holds E/64 logits and the
// wave finds the maximum k times with a butterfly reduction, ties going to
// the lower expert index. The weights are exp(l_j - l_max) in double
// precision, divided by their slot-order sum (renorm) or by the sum over all
// experts in ascending index order, and rounded once to fp32.
//
// Routing has to be bit-exact, and the pages name no exponential, so the
// weights are defined through one stated sequence of IEEE double operations
// (route_exp below): any implementation that follows the steps gets the same
// bits, on any device.
#include "moe_internal.h"

namespace moe {
namespace {

// exp(d) for d <= 0: 0 below -708 (and for -inf); otherwise Cody-Waite
// reduction d = n ln2 + r with n = rint(d / ln2) (ties to even, 1/ln2 as the
// nearest double), r = fma(-n, ln2_hi, d) then fma(-n, ln2_lo, r) with ln2_hi
// the double nearest ln 2 and ln2_lo the double nearest the remainder; then
// the Taylor polynomial sum over i <= 13 of r^i / i! in Horner form with fma,
// each coefficient the double nearest 1/i!; then times 2^n, exact for
// n >= -1021. Every step is one IEEE operation, written explicitly so that
// no contraction changes it.
__device__ double route_exp(double d) {
    if (!(d >= -708.0)) return 0.0;
    const double n = rint(d * 0x1.71547652b82fep+0);
    double r = fma(-n, 0x1.62e42fefa39efp-1, d);
    r = fma(-n, 0x1.abc9e3b39803fp-56, r);
    // 1/i! for i = 13 down to 0, each a correctly rounded quotient of exact
    // factorials
    constexpr double f[14] = {1.0, 1.0, 2.0, 6.0, 24.0, 120.0, 720.0, 5040.0, 40320.0, 362880.0, 3628800.0,
                              39916800.0, 479001600.0, 6227020800.0};
    double p = 1.0 / f[13];
#pragma unroll
    for (int i = 12; i >= 0; --i) p = fma(p, r, 1.0 / f[i]);
    return ldexp(p, (int)n);
}

__device__ __forceinline__ bool better(float a, int ea, float b, int eb) {
    return a > b || (a == b && ea < eb);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.T) return;  // the whole wave leaves together
    const float* row = p.logits + t * p.ls_t;
    float v[EPL];
    bool avail[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        int e = lane + kWave * i;
        avail[i] = e < p.E;
        v[i] = avail[i] ? row[(int64_t)e * p.ls_e] : -INFINITY;
    }
    float my_l = 0.0f;
    int my_e = 0;
    for (int j = 0; j < p.k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            int e = lane + kWave * i;
            if (avail[i] && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oe = __shfl_xor(be, off);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & (kWave - 1)) == lane) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (be >> 6)) avail[i] = false;
        }
        if (lane == j) {
            my_l = bv;
            my_e = be;
        }
    }
    const double m = (double)__shfl(my_l, 0);
    const double ex = route_exp((double)my_l - m);
    double denom = 0.0;
    if (p.renorm) {
        // slot order: ((e_0 + e_1) + e_2) + ...
        for (int j = 0; j < p.k; ++j) denom += __shfl(ex, j);
    } else {
        // every expert in ascending index order (expert e = lane + 64 i)
        double ev[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) ev[i] = lane + kWave * i < p.E ? route_exp((double)v[i] - m) : 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            for (int L = 0; L < kWave && L + kWave * i < p.E; ++L) denom += __shfl(ev[i], L);
    }
    if (lane < p.k) {
        p.ids[t * p.is_t + lane * p.is_j] = my_e;
        p.w[t * p.ws_t + lane * p.ws_j] = (float)(ex / denom);
    } else if (lane == p.k && p.shared_id >= 0) {
        p.ids[t * p.is_t + lane * p.is_j] = p.shared_id;
        p.w[t * p.ws_t + lane * p.ws_j] = p.shared_w;
    }
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    dim3 grid((unsigned)((p.T + 3) / 4)), block(256);
    const int epl = (p.E + kWave - 1) / kWave;
    if (epl <= 1)
        hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, p);
    else if (epl <= 2)
        hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, p);
    else if (epl <= 4)
        hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, p);
    else if (epl <= 8)
        hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
