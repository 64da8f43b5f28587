// Internal declarations shared by the HIP translation units of libmoeffn:
// device helpers (bf16 rounding, e2m1 coding, wave primitives) and the
// parameter blocks / launchers each kernel file exports to the host planner.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- types

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------- bf16 helpers

// Two fp32 -> two bf16 (low half = a), round to nearest even, with the
// chip's packed conversion (v_cvt_pk_bf16_f32; fp32 denormals are kept, the
// kernels' float mode): one instruction per pair, where a rounding written
// out in integer arithmetic took about six per value and bound the y
// epilogues. The bits equal the integer rounding for every finite value.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return (uint16_t)bf16x2_bits(f, 0.0f); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// SiLU(g) * u = g / (1 + e^-g) * u, the activation of every gemm1 epilogue
// (and of the backward's recompute): for very negative g, e^-g overflows to
// +inf and the reciprocal gives 0, so the result is a signed zero, never NaN.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __expf(-g);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ---------------------------------------------------------- e2m1 coding
//
// One group of 32 values shares the exponent s = floor(log2(amax)) - 2,
// clamped to [-127, 127] (s = -127 when amax is zero or subnormal). An
// element's code is the e2m1 magnitude nearest to |v| / 2^s, ties to the even
// code, saturating at 6. The decision is taken on the fp32 bit pattern of
// |v| against the seven midpoints scaled by 2^s, all integers, so it is exact
// whatever the denormal mode of the ALU.

// Shared exponent from the fp32 bits of amax (sign already cleared).
__device__ __forceinline__ int group_exponent(uint32_t amax_bits) {
    int ef = (int)(amax_bits >> 23);
    if (ef == 0) return -127;            // zero or subnormal: floor(log2) - 2 < -127
    int s = ef - 127 - 2;
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// fp32 bit pattern of mant * 2^e for mant in {1, 1.25, 1.5, 1.75} given as the
// 23-bit fraction; exact for every e >= -129 used here.
__device__ __forceinline__ uint32_t scaled_bits(uint32_t frac, int e) {
    if (e >= -126) return ((uint32_t)(e + 127) << 23) | frac;
    uint32_t full = (1u << 23) | frac;   // subnormal: value = full * 2^(e - 23)
    return full >> (-126 - e);
}

struct E2m1Thresholds {
    uint32_t t[7];
};

// Midpoints between neighbouring e2m1 magnitudes, scaled by 2^s:
// 0.25 0.75 1.25 1.75 2.5 3.5 5.
__device__ __forceinline__ E2m1Thresholds e2m1_thresholds(int s) {
    E2m1Thresholds th;
    th.t[0] = scaled_bits(0x000000u, s - 2);   // 1.0  * 2^-2
    th.t[1] = scaled_bits(0x400000u, s - 1);   // 1.5  * 2^-1
    th.t[2] = scaled_bits(0x200000u, s);       // 1.25 * 2^0
    th.t[3] = scaled_bits(0x600000u, s);       // 1.75 * 2^0
    th.t[4] = scaled_bits(0x200000u, s + 1);   // 1.25 * 2^1
    th.t[5] = scaled_bits(0x600000u, s + 1);   // 1.75 * 2^1
    th.t[6] = scaled_bits(0x200000u, s + 2);   // 1.25 * 2^2
    return th;
}

// Code of one value from its fp32 bits. At a midpoint whose lower neighbour
// has an odd code (0.75, 1.75, 3.5) the tie goes up to the even code.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t vbits, const E2m1Thresholds& th) {
    uint32_t a = vbits & 0x7fffffffu;
    uint32_t c = (a > th.t[0]) + (a >= th.t[1]) + (a > th.t[2]) + (a >= th.t[3]) +
                 (a > th.t[4]) + (a >= th.t[5]) + (a > th.t[6]);
    return c | ((vbits >> 28) & 8u);
}

// ------------------------------------------------------- wave primitives

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ------------------------------------------------------------- RMSNorm
//
// One summation order for every kernel that normalises a row (the norm
// kernels and the few-token gemm1 that folds the norm in): chunk c holds
// elements 8c .. 8c+7; lane q of one wave chains fmaf over the chunks
// c = q, q + 64, ... in ascending order, element by element; the 64 partials
// meet in a wave64 xor butterfly (distance 32, 16, ..., 1). The scale is
// then r = 1 / sqrt(ss / H + eps) and the output bf16((x * r) * w).

__device__ __forceinline__ float rms_scale(float ss, int64_t H, float eps) {
    return 1.0f / __builtin_sqrtf(ss / (float)H + eps);
}

// the two bf16 values of a 32-bit word, element order (low half first)
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Sum of squares of a bf16 row staged as nc 16-byte chunks (LDS), in the
// order above; call from one whole wave; every lane gets the sum.
__device__ __forceinline__ float row_sumsq_chunks(const uint4* row, int nc) {
    const int q = lane_id();
    float acc = 0.f;
    for (int c = q; c < nc; c += 64) {
        const uint4 v = row[c];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_lo(u[i]), hi = bf16_hi(u[i]);
            acc = __builtin_fmaf(lo, lo, acc);
            acc = __builtin_fmaf(hi, hi, acc);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
    return acc;
}

// Element h of the norm weight ([H], bf16 or fp32, element stride ws).
__device__ __forceinline__ float norm_weight_at(const void* w, bool f32, int64_t ws, int64_t h) {
    return f32 ? reinterpret_cast<const float*>(w)[h * ws]
               : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(w)[h * ws]);
}

// Workgroup index remapped so that consecutive logical tiles land on the same
// XCD: the hardware deals workgroups round-robin over the 8 XCDs, so block b
// runs on XCD b % 8. Logical index = (b % 8) * (G / 8) + b / 8 for the part of
// the grid that fills whole rounds; the tail keeps its index.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t G) {
    uint32_t full = G & ~7u;
    if (b >= full) return b;
    return (b & 7u) * (full >> 3) + (b >> 3);
}

// ------------------------------------------------------------ launchers

struct RouteParams {
    const float* logits;
    int64_t T, ls_t, ls_e;
    int32_t E, k, renorm, shared_id;
    float shared_w;
    int32_t* ids;
    int64_t is_t, is_j;
    float* w;
    int64_t ws_t, ws_j;
};
hipError_t launch_route(const RouteParams& p, hipStream_t s);

struct AlignParams {
    const int32_t* ids;
    int64_t is_t, is_j;
    int32_t T, k, A, E, bm;
    int64_t e_off;          // global id of local expert 0: slot ids are e_off + local
    int32_t cap, cap2;      // entries of sorted / sorted2 (every one is written)
    int32_t* sorted;        // [cap]
    int32_t* block_expert;  // [cap / bm]
    int32_t* n_padded;      // [1]
    int32_t* counts;        // [nchunks * E + 2 E] scratch (multi-block path)
    // optional second layout of the same order padded to bm2 (sorted2 null: none)
    int32_t bm2;
    int32_t* sorted2;
    int32_t* block_expert2;
    int32_t* n_padded2;
    // optional [E + 1]: first sorted block of each expert (entry E: the
    // block count), per layout (null: not written)
    int32_t* expert_block;
    int32_t* expert_block2;
};
// Scratch bytes the multi-block path needs for A assignments over E experts.
size_t align_scratch_bytes(int64_t A, int32_t E);
hipError_t launch_align(const AlignParams& p, hipStream_t s);
// The align with the activation preparation of kind (prep.h; 0: none) run by
// the spare workgroups of its first launch.
struct PrepParams;
hipError_t launch_align_prep(const AlignParams& p, int kind, const PrepParams& prep, hipStream_t s);
// The row-layout RMSNorm of prep.n (unit last-dim stride), then, with
// prep.quant_after, the MXFP4 quantisation prep.q of the normalised rows, as
// a launch of its own.
hipError_t launch_prep_norm_rows(const PrepParams& prep, hipStream_t s);

struct QuantParams {
    const uint16_t* src;
    int64_t ss_e, ss_r, ss_k;   // element strides
    uint8_t* codes;
    int64_t cs_e, cs_r;         // byte strides (last = 1)
    uint8_t* scales;
    int64_t xs_e, xs_r;
    int64_t E, R, K;            // leading count (1 for 2-D), rows, K
};
hipError_t launch_quant_mxfp4(const QuantParams& p, hipStream_t s);

// Quantise group g (32 consecutive values of one row) of p; g < E * R * K/32.
__device__ __forceinline__ void quant_group_mxfp4(const QuantParams& p, int64_t g) {
    const int64_t groups_per_row = p.K / 32;
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

struct PackParams {
    const uint16_t* src;
    int64_t s_t, s_h;
    uint16_t* dst;   // [T, H] contiguous
    int64_t T, H;
};
hipError_t launch_pack_bf16(const PackParams& p, hipStream_t s);

// RMSNorm of activation rows: out[t, h] = bf16((x[t, h] * r_t) * w[h]) with
// r_t = 1 / sqrt(sum_h x[t, h]^2 / H + eps); H a multiple of 8.
struct NormParams {
    const uint16_t* x;
    int64_t xs_t, xs_h;     // element strides
    const void* w;          // [H] bf16, or fp32 when w_f32
    int32_t w_f32;
    int64_t ws;             // element stride of w
    float eps;
    uint16_t* out;
    int64_t os_t, os_h;
    int64_t T, H;
};
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s);

// ------------------------------------------------------------- backward

// Rows of one GEMM operand. kind 0: row index in weight space (rows at or
// past split come from base[1]), expert e adds e * e_stride; kind 1: a sorted
// position, row = its token (a / k); kind 2: a sorted position, row = its
// assignment a. Sorted positions holding the sentinel read as zero rows.
struct BwdRowSrc {
    const uint16_t* base[2];
    int64_t e_stride[2], r_stride[2];   // elements
    int64_t split;
    int32_t kind;
};
struct BwdGemmParams {
    BwdRowSrc a, b;
    const int32_t* sorted;
    const int32_t* block_expert;
    const int32_t* n_padded;
    const int32_t* eb_first;   // first and last sorted block of each expert
    const int32_t* eb_last;
    int32_t A, k;
    int32_t K;                 // group 0: contraction length
    int32_t n_tiles, m_tiles;
    float* rows_out;           // group 0: fp32 rows by assignment
    int64_t rows_ld;
    void* out[2];              // group 1: weight gradients, rows at or past out_split in out[1]
    int64_t out_e[2], out_r[2];
    int64_t out_split;
    int32_t out_f32;
    int32_t out_accumulate;    // group 1: add into the existing values; experts without rows are skipped
};
hipError_t launch_bwd_gemm(int a_kmajor, int b_kmajor, int group, const BwdGemmParams& p, int64_t blocks,
                           hipStream_t s);
struct BwdActParams {
    const float* gu;           // [A, 2I] recomputed g | u
    const float* q;            // [A, I]
    uint16_t* dgu;             // [A, 2I] bf16 dg | du
    uint16_t* wh;              // [A, I] bf16 w * hb
    const int32_t* ids;
    int64_t is_t, is_j;
    const float* w;
    int64_t ws_t, ws_j;
    float* dw;
    int64_t dws_t, dws_j;
    int64_t e_off;
    int32_t E, k, I;
    int64_t A;
};
hipError_t launch_bwd_act(const BwdActParams& p, hipStream_t s);
struct BwdDxParams {
    const float* dxa;          // [A, H] per-slot dx
    const int32_t* ids;
    int64_t is_t, is_j;
    int64_t e_off;
    int32_t E, k;
    int64_t T, H;
    uint16_t* dx;
    int64_t os_t, os_h;
};
hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s);
hipError_t launch_bwd_expert_blocks(const int32_t* block_expert, const int32_t* n_padded, int bm, int max_blocks,
                                    int32_t* first, int32_t* last, int E, hipStream_t s);

// One grouped GEMM launch. Stage 1: A = gathered x rows, B = gate/up rows,
// epilogue SiLU(g)*u -> h. Stage 2: A = h rows, B = w2 rows, epilogue scatter
// of y rows (fp32; bf16 in MXFP4 mode) to their flat assignment index.
struct GemmParams {
    // routing / align
    const int32_t* sorted;
    const int32_t* block_expert;
    const int32_t* n_padded;
    int32_t A, k, E;
    // A operand
    const void* a;          // bf16 [rows, K] or fp4x2 [rows, K/2]
    int64_t a_row;          // row stride in elements (bf16) or bytes (fp4)
    const uint8_t* a_sc;    // fp4 scales [rows, K/32]
    int64_t a_sc_row;
    // B operands (weights); for stage 1 b0 = gate, b1 = up, for stage 2 b0 = w2
    const void* b0;
    const void* b1;
    int64_t b0_e, b0_r, b1_e, b1_r;          // strides: elements (bf16) / bytes (fp4)
    const uint8_t* b0_sc;
    const uint8_t* b1_sc;
    int64_t b0sc_e, b0sc_r, b1sc_e, b1sc_r;  // scale strides in bytes
    int32_t K;              // contraction length
    int32_t N;              // output columns (stage 1: I, stage 2: H)
    // outputs
    void* out;              // stage 1: h (bf16 [A, I] or fp4 [A, I/2]); stage 2: y (bf16 rows of out_row
                            // elements); both by flat assignment index
    int64_t out_row;        // stage 2: element stride between y rows
    uint8_t* out_sc;        // stage 1 MXFP4: h scales [A, I/32]
    int32_t n_tile_groups;  // tiles along N are walked in groups of this size
    int32_t max_mblocks;
    const int32_t* expert_block;   // [E + 1] first sorted block of each expert (LDS-tiled kernels)
};

struct GemmKernelId {
    int mode;    // 0 bf16, 1 mxfp4
    int stage;   // 1 or 2
    int bm;      // 16, 32, 64
    int wk;      // waves splitting K: 1, 2 or 4
    int u;       // weight steps in each wave's load ring (from gemm_ring_steps)
    int nb;      // 16-column MFMA blocks per wave: 4, or 2 (bf16 weight stream)
    int nt = 1;  // MXFP4 gemm2 with K = 512: 256-column tiles per workgroup (1, 2, 4, 8)
};
// Ring depth for a wave's share of K.
int gemm_ring_steps(int mode, int bm, int nb, int wk, int64_t k_per_wave);
// Output columns one workgroup covers.
int gemm_tile_n(const GemmKernelId& id);
// Smallest unit of K a wave's share must be a multiple of.
int gemm_k_granule(const GemmKernelId& id);
bool gemm_supported(const GemmKernelId& id);
hipError_t launch_gemm(const GemmKernelId& id, const GemmParams& p, hipStream_t s);

// LDS-tiled grouped GEMM. Tile shapes (rows x weight rows per workgroup):
// 0 = 256 x 256, 1 = 128 x 512 (bf16 only), 2 = 64 x 512, 3 = 32 x 512,
// 4 = 64 x 256 (bf16) / 32 x 256 (MXFP4), 5 = 128 x 256.
// Row blocks of gemm_tile_rows(mode, shape), gemm_tile_cols(shape, stage) output
// columns per workgroup, K a multiple of gemm_tile_k_granule(mode, shape). Same
// parameter block and epilogues as above.
// Shapes 6 and 7 (MXFP4 gemm2 with K = 512 only): a workgroup keeps 256 or
// 128 h rows in registers and walks the output columns in 128-wide weight
// tiles (gemm2_rows.hip); y stored with 32-bit buffer offsets, so the y rows
// must span less than 4 GB.
bool gemm2_rows_supported(int64_t K, int64_t N, int64_t A, int64_t out_row);
hipError_t launch_gemm2_rows(int bm, const GemmParams& p, hipStream_t s);
int gemm_tile_rows(int mode, int shape);
int gemm_tile_cols(int shape, int stage);
int gemm_tile_k_granule(int mode, int shape);
bool gemm_tile_supported(int mode, int shape);
hipError_t launch_gemm_tile(int mode, int shape, int stage, const GemmParams& p, hipStream_t s);

struct CombineParams {
    const uint16_t* y;      // bf16 row of slot (t, j) at t * ys_t + j * ys_j
    int64_t ys_t, ys_j;
    int64_t e_off;          // slot counts when 0 <= id - e_off < E
    const int32_t* ids;
    int64_t is_t, is_j;
    const float* w;
    int64_t ws_t, ws_j;
    uint16_t* out;
    int64_t os_t, os_h;
    int32_t T, k, E, H;
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

// MXFP4 gemm2 with the combine folded in, for a few tokens: g describes
// gemm2 (h codes and scales by flat assignment, w2, K = 512), c the combine.
struct Gemm2CombineParams {
    GemmParams g;
    CombineParams c;
};
hipError_t launch_gemm2_combine(const Gemm2CombineParams& p, hipStream_t s);

// MXFP4 gemm1 for a few tokens without the align: one workgroup per (slot,
// 32 h columns); the expert comes from the ids, the activation row is
// quantised into LDS. Writes h codes and scales by flat assignment.
struct Gemm1SmallParams {
    const uint16_t* x;          // bf16 activation rows
    int64_t xs_t, xs_h;
    const uint8_t* gate;        // fp4x2 codes and e8m0 scales, byte strides
    const uint8_t* up;
    int64_t g_e, g_r, u_e, u_r;
    const uint8_t* gate_sc;
    const uint8_t* up_sc;
    int64_t gs_e, gs_r, us_e, us_r;
    const int32_t* ids;
    int64_t is_t, is_j;
    int64_t e_off;
    int32_t E, k, A, H, I;
    uint8_t* hq;                // [A, I/2]
    uint8_t* hs;                // [A, I/32]
    // RMSNorm folded in (nw null: off): the token row is normalised in LDS
    // in the norm kernels' order before it is used, bit-identical to the
    // separate pass
    const void* nw;             // [H] bf16, or fp32 when nw_f32
    int64_t nws;                // element stride of nw
    int32_t nw_f32;
    float eps;
};
hipError_t launch_gemm1_small(const Gemm1SmallParams& p, hipStream_t s);
// the same in bf16: h bf16 [A, I] in hq (byte strides for the weights)
hipError_t launch_gemm1_small_bf16(const Gemm1SmallParams& p, hipStream_t s);
// bf16 gemm2 (K split 4 inside the workgroup) with the combine folded in;
// K = I a multiple of 256 from 512 to 1536
bool gemm2_combine_bf16_supported(int64_t I);
hipError_t launch_gemm2_combine_bf16(const Gemm2CombineParams& p, hipStream_t s);

// Record "what: detail" as the calling thread's moe_last_error() text and
// return status (for entry points outside the host planner's file).
int report_error(int status, const char* what, const char* detail);

}  // namespace moe
