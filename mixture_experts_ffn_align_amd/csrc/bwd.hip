// Backward of the bf16 fused forward: the gradients of L = sum(dout * out)
// with respect to x, the top-k weights, gate, up and w2 (Liger-Kernel PR
// #1377, Notes: the grad-enabled path of the same fused MoE, whose inputs
// follow the same stride rules).
//
// Per valid slot a = (t, j) of expert e, with h and its bf16 rounding hb
// exactly as the forward computes them:
//   g, u  = gate_e x_t, up_e x_t              (recomputed, fp32)
//   q     = w2_e^T dout_t                     (q_i = sum_n dout_n w2[n, i])
//   dw_tj = <q, hb>  (= <dout_t, y_tj>, y = w2_e hb)
//   dh    = w_tj q,  dg = dh u SiLU'(g),  du = dh SiLU(g)
//   dx_t  = sum over j of (gate_e^T dg + up_e^T du)
//   dW2_e = sum over a of dout_t (w hb)^T,  dG_e = sum dg x_t^T,  dU_e = sum du x_t^T
// dg, du and w hb enter the later GEMMs rounded to bf16. Sums over slots and
// over an expert's rows run in a fixed order, so results do not vary from
// run to run.
//
// One MFMA kernel serves all five GEMMs: BM x 128 output tiles (BM 64 over
// sorted row blocks, 128 over weight space), 4 waves of BM/2 x 64, K in
// stages of 64 staged through LDS in rows of 128 bytes (K contiguous, 16-byte
// chunks XOR-swizzled by the row). An operand is read either by rows (K
// contiguous in memory: activations, gate/up rows) or K-major (rows of memory
// are K: w2 rows for q, gate/up rows for dx, all activations for the weight
// gradients); a K-major stage is loaded by every thread as a 4 x 8 block and
// transposed in registers before it is written to LDS.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBN = 128, kBK = 64;
constexpr int kRowB = kBK * 2;                       // bytes per LDS tile row

__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

// Element 0 of row idx of a source, or null for a padding row.
__device__ __forceinline__ const uint16_t* src_row(const BwdRowSrc& s, const BwdGemmParams& p, int64_t idx, int e) {
    if (s.kind == 0) {
        const int h = idx >= s.split ? 1 : 0;
        return s.base[h] + (int64_t)e * s.e_stride[h] + (idx - (h ? s.split : 0)) * s.r_stride[h];
    }
    const int a = p.sorted[idx];
    if (a >= p.A) return nullptr;
    return s.base[0] + (int64_t)(s.kind == 1 ? a / p.k : a) * s.r_stride[0];
}

__device__ __forceinline__ uint4 load16(const uint16_t* ptr) {
    return ptr ? *reinterpret_cast<const uint4*>(ptr) : make_uint4(0u, 0u, 0u, 0u);
}

// 4 x 8 bf16 block: v[i] holds 8 consecutive columns of row i; entry c of
// the result holds rows 0..3 of column c.
__device__ __forceinline__ void transpose4x8(const uint4 (&v)[4], uint2 (&o)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t lo = (&v[2 * q].x)[c >> 1], hi = (&v[2 * q + 1].x)[c >> 1];
            w[q] = __builtin_amdgcn_perm(hi, lo, sel);
        }
        o[c] = make_uint2(w[0], w[1]);
    }
}

// One operand's share of a stage in registers. ROWS: R rows x 8 chunks over
// 256 threads. KMAJOR (R = 128): thread u owns k rows 4 (u % 16) .. + 3 of
// columns 8 (u / 16) .. + 7.
template <int MODE, int R>
struct Stage {
    static_assert(MODE == 0 || R == 128, "K-major operands are 128 columns wide");
    static constexpr int kRowsN = MODE == 0 ? R * 8 / 256 : 4;
    uint4 v[kRowsN];
};

template <int MODE, int R>
struct Operand {
    const BwdRowSrc* s;
    int e;
    int64_t col0;                        // KMAJOR: first column of the tile
    const uint16_t* rows[MODE == 0 ? R * 8 / 256 : 1];   // ROWS: resolved once
    int32_t ent[4];                      // KMAJOR over sorted positions: the next stage's entries

    __device__ void init(const BwdRowSrc& src, const BwdGemmParams& p, int e_, int64_t row0, int64_t c0) {
        s = &src;
        e = e_;
        col0 = c0;
        if constexpr (MODE == 0) {
#pragma unroll
            for (int j = 0; j < R * 8 / 256; ++j) {
                const int idx = threadIdx.x + 256 * j;
                rows[j] = src_row(src, p, row0 + (idx >> 3), e);
            }
        }
    }
    // KMAJOR over sorted positions: fetch the sorted entries of the stage
    // whose k rows start at kidx one stage ahead of its loads
    __device__ void prep(const BwdGemmParams& p, int64_t kidx) {
        if constexpr (MODE == 1) {
            if (s->kind != 0) {
                const int kq = threadIdx.x & 15;
#pragma unroll
                for (int i = 0; i < 4; ++i) ent[i] = p.sorted[kidx + 4 * kq + i];
            }
        }
    }
    // k rows start at kidx (a K index of the source for KMAJOR, an offset
    // into the rows for ROWS); KMAJOR over sorted positions uses the entries
    // prep fetched for this stage
    __device__ void load(const BwdGemmParams& p, int64_t kidx, Stage<MODE, R>& st) const {
        if constexpr (MODE == 0) {
#pragma unroll
            for (int j = 0; j < R * 8 / 256; ++j) {
                const int ch = (threadIdx.x + 256 * j) & 7;
                st.v[j] = load16(rows[j] ? rows[j] + kidx + 8 * ch : nullptr);
            }
        } else {
            const int u = threadIdx.x;
            const int kq = u & 15, cg = u >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t* r;
                if (s->kind == 0) {
                    r = src_row(*s, p, kidx + 4 * kq + i, e);
                } else {
                    const int a = ent[i];
                    r = a < p.A ? s->base[0] + (int64_t)(s->kind == 1 ? a / p.k : a) * s->r_stride[0] : nullptr;
                }
                st.v[i] = load16(r ? r + col0 + 8 * cg : nullptr);
            }
        }
    }
    __device__ void store(char* tile, const Stage<MODE, R>& st) const {
        if constexpr (MODE == 0) {
#pragma unroll
            for (int j = 0; j < R * 8 / 256; ++j) {
                const int idx = threadIdx.x + 256 * j, r = idx >> 3, ch = idx & 7;
                *reinterpret_cast<uint4*>(tile + r * kRowB + swz(r, ch) * 16) = st.v[j];
            }
        } else {
            const int u = threadIdx.x;
            const int kq = u & 15, cg = u >> 4;
            uint2 o[8];
            transpose4x8(st.v, o);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int r = 8 * cg + c;
                *reinterpret_cast<uint2*>(tile + r * kRowB + swz(r, kq >> 1) * 16 + (kq & 1) * 8) = o[c];
            }
        }
    }
};

// A: M x K, B: N x K in LDS; C[m, n] = sum_k A[m, k] B[n, k].
// G = 0: M runs over 64 sorted rows of one expert (rows_out by assignment);
// G = 1: M, N over weight space (BM = 128), K over the expert's sorted rows.
template <int AM, int BMODE, int G>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemmParams p) {
    constexpr int kBM = G == 0 ? 64 : 128;
    constexpr int kMB = kBM / 32;                    // 16-row blocks per wave
    __shared__ __attribute__((aligned(16))) char lds[2][(kBM + kBN) * kRowB];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w & 1, wn = w >> 1;
    const int nt = blockIdx.x % p.n_tiles;
    int e, S;
    int64_t m0, kb0 = 0;
    if constexpr (G == 0) {
        const int blk = blockIdx.x / p.n_tiles;
        if (blk * kBM >= *p.n_padded) return;
        e = p.block_expert[blk];
        m0 = (int64_t)blk * kBM;
        S = p.K / kBK;
    } else {
        const int rest = blockIdx.x / p.n_tiles;
        const int mt = rest % p.m_tiles;
        e = rest / p.m_tiles;
        m0 = (int64_t)mt * kBM;
        const int first = p.eb_first[e];
        S = p.eb_last[e] - first + 1;
        kb0 = (int64_t)first * kBK;
        if (p.out_accumulate && S <= 0) return;   // nothing to add
    }
    const int64_t n0 = (int64_t)nt * kBN;
    Operand<AM, kBM> A;
    Operand<BMODE, kBN> B;
    // ROWS operands name their rows once (sorted positions or weight rows);
    // KMAJOR operands name a column range and read K rows per stage
    A.init(p.a, p, e, m0, m0);
    B.init(p.b, p, e, n0, n0);
    auto kidx = [&](int s) -> int64_t { return G == 0 ? (int64_t)s * kBK : kb0 + (int64_t)s * kBK; };

    f32x4_t acc[4][kMB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kMB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Stage<AM, kBM> sa;
    Stage<BMODE, kBN> sb;
    if (S > 0) {
        A.prep(p, kidx(0));
        B.prep(p, kidx(0));
        A.load(p, AM == 0 ? 0 : kidx(0), sa);
        B.load(p, BMODE == 0 ? 0 : kidx(0), sb);
        if (S > 1) {
            A.prep(p, kidx(1));
            B.prep(p, kidx(1));
        }
        A.store(lds[0], sa);
        B.store(lds[0] + kBM * kRowB, sb);
    }
    __syncthreads();
    for (int s = 0; s < S; ++s) {
        const bool more = s + 1 < S;
        if (more) {
            A.load(p, AM == 0 ? (int64_t)(s + 1) * kBK : kidx(s + 1), sa);
            B.load(p, BMODE == 0 ? (int64_t)(s + 1) * kBK : kidx(s + 1), sb);
            if (s + 2 < S) {
                A.prep(p, kidx(s + 2));
                B.prep(p, kidx(s + 2));
            }
        }
        const char* ta = lds[s & 1];
        const char* tb = ta + kBM * kRowB;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ck = ks * 4 + (lane >> 4);
            uint4 fa[kMB], fb[4];
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) {
                const int r = wm * (kBM / 2) + mb * 16 + (lane & 15);
                fa[mb] = *reinterpret_cast<const uint4*>(ta + r * kRowB + swz(r, ck) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int r = wn * 64 + nb * 16 + (lane & 15);
                fb[nb] = *reinterpret_cast<const uint4*>(tb + r * kRowB + swz(r, ck) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, fb[nb]), __builtin_bit_cast(bf16x8_t, fa[mb]), acc[nb][mb], 0,
                        0, 0);
        }
        if (more) {
            A.store(lds[(s + 1) & 1], sa);
            B.store(lds[(s + 1) & 1] + kBM * kRowB, sb);
        }
        __syncthreads();
    }
    // lane holds C[m = wm BM/2 + mb 16 + lane % 16][n = wn 64 + nb 16 + 4 (lane / 16) + i]
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
        const int m = wm * (kBM / 2) + mb * 16 + (lane & 15);
        if constexpr (G == 0) {
            const int a = p.sorted[m0 + m];
            if (a >= p.A) continue;
            float* row = p.rows_out + (int64_t)a * p.rows_ld + n0 + wn * 64 + 4 * (lane >> 4);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) *reinterpret_cast<f32x4_t*>(row + nb * 16) = acc[nb][mb];
        } else {
            const int64_t mm = m0 + m;
            const int h = mm >= p.out_split ? 1 : 0;
            const int64_t off = (int64_t)e * p.out_e[h] + (mm - (h ? p.out_split : 0)) * p.out_r[h] + n0 + wn * 64 +
                                4 * (lane >> 4);
            if (p.out_f32) {
                float* row = reinterpret_cast<float*>(p.out[h]) + off;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    f32x4_t v = acc[nb][mb];
                    if (p.out_accumulate) v = *reinterpret_cast<const f32x4_t*>(row + nb * 16) + v;
                    *reinterpret_cast<f32x4_t*>(row + nb * 16) = v;
                }
            } else {
                uint16_t* row = reinterpret_cast<uint16_t*>(p.out[h]) + off;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    f32x4_t v = acc[nb][mb];
                    if (p.out_accumulate) {
                        const uint2 o = *reinterpret_cast<const uint2*>(row + nb * 16);
                        v[0] = __uint_as_float(o.x << 16) + v[0];
                        v[1] = __uint_as_float(o.x & 0xffff0000u) + v[1];
                        v[2] = __uint_as_float(o.y << 16) + v[2];
                        v[3] = __uint_as_float(o.y & 0xffff0000u) + v[3];
                    }
                    *reinterpret_cast<uint2*>(row + nb * 16) =
                        make_uint2(bf16x2_bits(v[0], v[1]),
                                   bf16x2_bits(v[2], v[3]));
                }
            }
        }
    }
}

// Per slot: hb, dw, dg, du and w hb from the recomputed g, u and from q; one
// wave per slot, 4 consecutive columns per lane and step.
__global__ __launch_bounds__(256) void bwd_act_kernel(BwdActParams p) {
    const int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (a >= p.A) return;
    const int lane = threadIdx.x & 63;
    const int64_t t = a / p.k, j = a % p.k;
    const int64_t e = (int64_t)p.ids[t * p.is_t + j * p.is_j] - p.e_off;
    float* dwp = p.dw + t * p.dws_t + j * p.dws_j;
    if (e < 0 || e >= p.E) {
        if (lane == 0) *dwp = 0.f;
        return;
    }
    const float wt = p.w[t * p.ws_t + j * p.ws_j];
    const int64_t I = p.I;
    const float* gu = p.gu + a * 2 * I;
    const float* q = p.q + a * I;
    uint16_t* dgu = p.dgu + a * 2 * I;
    uint16_t* wh = p.wh + a * I;
    float acc = 0.f;
    for (int64_t i = 4 * lane; i < I; i += 256) {
        const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(gu + i);
        const f32x4_t u4 = *reinterpret_cast<const f32x4_t*>(gu + I + i);
        const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(q + i);
        uint32_t dg[4], du[4], hw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float g = g4[c], u = u4[c], qv = q4[c];
            const float hb = bf16_bits_to_f32(f32_to_bf16_bits(silu_mul(g, u)));
            acc = __builtin_fmaf(qv, hb, acc);
            const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
            const float dh = wt * qv;
            dg[c] = f32_to_bf16_bits(dh * u * (s * (1.0f + g * (1.0f - s))));
            du[c] = f32_to_bf16_bits(dh * (g * s));
            hw[c] = f32_to_bf16_bits(wt * hb);
        }
        *reinterpret_cast<uint2*>(dgu + i) = make_uint2(dg[0] | (dg[1] << 16), dg[2] | (dg[3] << 16));
        *reinterpret_cast<uint2*>(dgu + I + i) = make_uint2(du[0] | (du[1] << 16), du[2] | (du[3] << 16));
        *reinterpret_cast<uint2*>(wh + i) = make_uint2(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
    if (lane == 0) *dwp = acc;
}

// dx[t, n] = bf16(sum over valid slots j, in order, of dxa[t k + j, n]); 8
// columns per thread.
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdDxParams p) {
    const int ncol = p.H / 8;
    const int nqb = (ncol + 255) / 256;
    const int64_t total = p.T * nqb;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t t = b / nqb;
        const int q = (int)(b % nqb) * 256 + threadIdx.x;
        if (q >= ncol) continue;
        const int64_t n = (int64_t)q * 8;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j < p.k; ++j) {
            const int64_t e = (int64_t)p.ids[t * p.is_t + (int64_t)j * p.is_j] - p.e_off;
            if (e < 0 || e >= p.E) continue;
            const float* src = p.dxa + (t * p.k + j) * p.H + n;
            const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(src);
            const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] += v0[i];
                acc[4 + i] += v1[i];
            }
        }
        uint16_t* o = p.dx + t * p.os_t;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[(n + i) * p.os_h] = f32_to_bf16_bits(acc[i]);
    }
}

// First and last sorted block of every expert (first 0, last -1 when none).
__global__ __launch_bounds__(256) void bwd_eb_init_kernel(int32_t* first, int32_t* last, int E) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < E) {
        first[i] = 0;
        last[i] = -1;
    }
}

__global__ __launch_bounds__(256) void bwd_eb_mark_kernel(const int32_t* block_expert, const int32_t* n_padded,
                                                          int bm, int max_blocks, int32_t* first, int32_t* last) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    const int nb = *n_padded / bm;
    if (b >= nb || b >= max_blocks) return;
    const int e = block_expert[b];
    if (b == 0 || block_expert[b - 1] != e) first[e] = b;
    if (b == nb - 1 || block_expert[b + 1] != e) last[e] = b;
}

}  // namespace

hipError_t launch_bwd_gemm(int a_kmajor, int b_kmajor, int group, const BwdGemmParams& p, int64_t blocks,
                           hipStream_t s) {
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
    if (group == 0 && !a_kmajor && !b_kmajor) hipLaunchKernelGGL((bwd_gemm_kernel<0, 0, 0>), grid, block, 0, s, p);
    else if (group == 0 && !a_kmajor && b_kmajor) hipLaunchKernelGGL((bwd_gemm_kernel<0, 1, 0>), grid, block, 0, s, p);
    else if (group == 1 && a_kmajor && b_kmajor) hipLaunchKernelGGL((bwd_gemm_kernel<1, 1, 1>), grid, block, 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_bwd_act(const BwdActParams& p, hipStream_t s) {
    if (p.A == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_act_kernel, dim3((unsigned)((p.A + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s) {
    if (p.T == 0) return hipSuccess;
    const int64_t blocks = ((p.H / 8 + 255) / 256) * p.T;
    hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)std::min<int64_t>(blocks, (int64_t)1 << 22)), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

hipError_t launch_bwd_expert_blocks(const int32_t* block_expert, const int32_t* n_padded, int bm, int max_blocks,
                                    int32_t* first, int32_t* last, int E, hipStream_t s) {
    hipLaunchKernelGGL(bwd_eb_init_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, first, last, E);
    if (max_blocks > 0)
        hipLaunchKernelGGL(bwd_eb_mark_kernel, dim3((unsigned)((max_blocks + 255) / 256)), dim3(256), 0, s,
                           block_expert, n_padded, bm, max_blocks, first, last);
    return hipGetLastError();
}

}  // namespace moe
