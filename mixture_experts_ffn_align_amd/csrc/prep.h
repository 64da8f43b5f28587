// Activation preparation ahead of gemm1, as workgroup bodies shared by the
// standalone kernels (moe_rmsnorm, the re-layout and quantisation launches)
// and by the fused forward, where the spare workgroups of the align launch
// run them next to the sort (the norm of a re-laid-out x follows in a launch
// of its own, since it needs the whole re-laid-out row):
//  - RMSNorm of the token rows (LightLLM issue #1467, Summary and Expected
//    Behavior: the variance and the normalize pass both read the row through
//    its last-dim stride; the normalised row is multiplied by the weight):
//      out[t, h] = bf16( (x[t, h] * r_t) * w[h] ),  r_t = 1 / sqrt(ss_t / H + eps);
//  - the bf16 re-layout of an activation whose rows are not 16-byte runs
//    (last-dim stride != 1: read through its strides, never as if contiguous);
//  - the MXFP4 quantisation of the (normalised) rows.
//
// The sum of squares has one fixed order for every layout and every body
// (see the RMSNorm helpers in moe_internal.h), so a transposed activation
// gives the same bits as a contiguous one, and a body gives the same bits
// whichever launch runs it.
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- RMSNorm

__device__ __forceinline__ float prep_norm_weight(const NormParams& p, int64_t h) {
    return norm_weight_at(p.w, p.w_f32 != 0, p.ws, h);
}

// The 8 values of chunk c of row xr.
__device__ __forceinline__ void prep_load_chunk(const uint16_t* xr, int64_t s_h, bool vec, int64_t c,
                                                float (&v)[8]) {
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

__device__ __forceinline__ bool prep_weights_vec(const NormParams& p) {
    return p.ws == 1 && (((uintptr_t)p.w) & 15u) == 0;
}

// The 8 weights of chunk c (one or two 16-byte loads when w is contiguous
// and aligned).
__device__ __forceinline__ void prep_load_weights(const NormParams& p, bool wvec, int64_t c, float (&wv)[8]) {
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
        for (int i = 0; i < 8; ++i) wv[i] = prep_norm_weight(p, 8 * c + i);
    }
}

// Normalised chunk c of a row to the output row dr (element stride os_h).
__device__ __forceinline__ void prep_store_chunk(const NormParams& p, const float (&v)[8], const float (&wv)[8],
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

// Row t (unit last-dim stride), by one whole wave: lane q owns partial q.
// With NCL > 0 (H <= 512 NCL) a lane loads all its chunks and their weights
// at once and keeps them in registers for the second pass (every load of the
// row before any store: stores share the load counter, and a wait for a
// later load would also wait for them); NCL = 0 loops and reads the row
// twice. Both give the same bits.
template <int NCL>
__device__ __forceinline__ void prep_norm_row(const NormParams& p, int64_t t, int q) {
    const uint16_t* xr = p.x + t * p.xs_t;
    const bool vec = (((uintptr_t)xr) & 15u) == 0;
    const int64_t nc = p.H / 8;
    uint16_t* dr = p.out + t * p.os_t;
    float acc = 0.f;
    const bool wvec = prep_weights_vec(p);
    if constexpr (NCL > 0) {
        float v[NCL][8], wv[NCL][8];
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int64_t c = q + 64 * j;
            if (c < nc) {
                prep_load_chunk(xr, 1, vec, c, v[j]);
                prep_load_weights(p, wvec, c, wv[j]);
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
            if (c < nc) prep_store_chunk(p, v[j], wv[j], r, c, dr);
        }
    } else {
        for (int64_t c = q; c < nc; c += 64) {
            float v[8];
            prep_load_chunk(xr, 1, vec, c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[i], v[i], acc);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
        const float r = rms_scale(acc, p.H, p.eps);
        for (int64_t c = q; c < nc; c += 64) {
            float v[8], wv[8];
            prep_load_chunk(xr, 1, vec, c, v);
            prep_load_weights(p, wvec, c, wv);
            prep_store_chunk(p, v, wv, r, c, dr);
        }
    }
}

// LDS of one column-layout norm workgroup
struct PrepNormColsLds {
    float part[64][65];
    float scale[64];
};

// Any strides: rows 64 bx .. +64 by a workgroup of NW waves, lane = row (an
// activation stored transposed, s_t = 1, is read with unit stride across the
// lanes). Wave w computes partials q = w, w + NW, ... of every row, each with
// the 8 chunks c = q + 64 j of a group loaded at once; the partials meet in
// LDS and wave 0 adds them in the butterfly's pairing; then the waves
// normalise chunks c = NW y + w + NW S j (y = by of S column slices; S > 1
// spreads the stores of few rows over more CUs, each slice recomputing the
// sums), loading 4 chunks before storing them. Every thread reaches both
// barriers.
template <int NW>
__device__ __forceinline__ void prep_norm_cols(const NormParams& p, int64_t bx, int by, int S, PrepNormColsLds& L) {
    static_assert(64 % NW == 0, "waves divide the 64 partials");
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = bx * 64 + lane;
    const bool live = t < p.T;
    const uint16_t* xr = p.x + (live ? t : 0) * p.xs_t;
    const int64_t nc = p.H / 8;
#pragma unroll 1
    for (int qi = 0; qi < 64 / NW; ++qi) {
        const int q = w + NW * qi;
        float acc = 0.f;
#pragma unroll 1
        for (int64_t c0 = q; c0 < nc; c0 += 64 * 8) {
            float v[8][8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + 64 * j < nc) prep_load_chunk(xr, p.xs_h, false, c0 + 64 * j, v[j]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + 64 * j < nc) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[j][i], v[j][i], acc);
                }
            }
        }
        L.part[q][lane] = acc;
    }
    __syncthreads();
    if (w == 0) {
        float v[64];
#pragma unroll
        for (int q = 0; q < 64; ++q) v[q] = L.part[q][lane];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int q = 0; q < m; ++q) v[q] = v[q] + v[q + m];
        }
        L.scale[lane] = rms_scale(v[0], p.H, p.eps);
    }
    __syncthreads();
    if (!live) return;
    const float r = L.scale[lane];
    uint16_t* dr = p.out + t * p.os_t;
    const bool wvec = prep_weights_vec(p);
    const int64_t step = NW * (int64_t)S;
#pragma unroll 1
    for (int64_t c0 = NW * (int64_t)by + w; c0 < nc; c0 += 4 * step) {
        float v[4][8], wv[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = c0 + step * j;
            if (c < nc) {
                prep_load_chunk(xr, p.xs_h, false, c, v[j]);
                prep_load_weights(p, wvec, c, wv[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = c0 + step * j;
            if (c < nc) prep_store_chunk(p, v[j], wv[j], r, c, dr);
        }
    }
}

// -------------------------------------------------------- bf16 re-layout

// dst[t, h] = src[t*s_t + h*s_h]: a group of 256 threads moves one 64-token x
// 64-column tile through LDS. Lanes walk t on the read side, so an activation
// stored transposed (s_t = 1) is read in 128-byte runs, and eight lanes write
// each destination row's 128 bytes on the store side, so every store fills
// whole cache lines. Load, then a workgroup barrier, then store.
constexpr int kPackTile = 64;
typedef uint16_t PackTileLds[kPackTile][kPackTile + 8];

__device__ __forceinline__ void prep_pack_load(const PackParams& p, int64_t t0, int64_t h0, int tid,
                                               PackTileLds& tile) {
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll 4
    for (int i = 0; i < kPackTile / 4; ++i) {
        const int hl = i * 4 + wv;
        const int64_t t = t0 + lane, h = h0 + hl;
        if (t < p.T && h < p.H) tile[lane][hl] = p.src[t * p.s_t + h * p.s_h];
    }
}

__device__ __forceinline__ void prep_pack_store(const PackParams& p, int64_t t0, int64_t h0, int tid,
                                                const PackTileLds& tile) {
    const int chunk = tid & 7;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int tl = (tid >> 3) + 32 * pass;
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

// ------------------------------------------- preparation inside the align

// What the spare workgroups of the align launch do (kind), and on what.
enum PrepKind : int {
    kPrepQuant = 1,      // MXFP4 quantisation of x, one thread per 32-group
    kPrepPack = 2,       // bf16 re-layout of a strided x
    kPrepNormRows = 3,   // RMSNorm, unit last-dim stride: one wave per row
};
struct PrepParams {
    QuantParams q;     // kPrepQuant; with a norm kind and quant_after, src = the normalised rows
    PackParams pk;
    NormParams n;
    int32_t quant_after;   // kPrepNormRows: quantise the workgroup's normalised rows next
    int64_t blocks;        // workgroups the preparation needs
};

// Workgroups of NT threads that the preparation of kind K needs.
inline int64_t prep_blocks(int kind, const PrepParams& pr, int nt) {
    switch (kind) {
    case kPrepQuant: return (pr.q.E * pr.q.R * (pr.q.K / 32) + nt - 1) / nt;
    case kPrepPack: {
        const int64_t tiles = ((pr.pk.T + kPackTile - 1) / kPackTile) * ((pr.pk.H + kPackTile - 1) / kPackTile);
        const int64_t per = nt / 256;
        return (tiles + per - 1) / per;
    }
    case kPrepNormRows: return (pr.n.T + nt / 64 - 1) / (nt / 64);
    default: return 0;
    }
}

// Preparation workgroup b (0-based among the spare ones) of NT threads.
template <int KIND, int NCL, int NT>
__device__ __forceinline__ void prep_block(const PrepParams& pr, int64_t b) {
    const int tid = threadIdx.x;
    if constexpr (KIND == kPrepQuant) {
        const int64_t g = b * NT + tid;
        if (g < pr.q.E * pr.q.R * (pr.q.K / 32)) quant_group_mxfp4(pr.q, g);
    } else if constexpr (KIND == kPrepPack) {
        constexpr int kPer = NT / 256;
        __shared__ PackTileLds tiles[kPer];
        const int sub = tid >> 8;
        const int64_t ntt = (pr.pk.T + kPackTile - 1) / kPackTile;
        const int64_t nth = (pr.pk.H + kPackTile - 1) / kPackTile;
        const int64_t ti = b * kPer + sub;
        const bool live = ti < ntt * nth;
        const int64_t t0 = (ti % ntt) * kPackTile, h0 = (ti / ntt) * kPackTile;
        if (live) prep_pack_load(pr.pk, t0, h0, tid & 255, tiles[sub]);
        __syncthreads();
        if (live) prep_pack_store(pr.pk, t0, h0, tid & 255, tiles[sub]);
    } else {
        static_assert(KIND == kPrepNormRows, "preparation kind");
        // rows [r0, r0 + NT / 64), one per wave
        const int64_t r0 = b * (NT / 64);
        const int64_t t = r0 + (tid >> 6);
        if (t < pr.n.T) prep_norm_row<NCL>(pr.n, t, tid & 63);
        if (pr.quant_after) {
            // the normalised rows were written by this workgroup: a
            // workgroup barrier orders those stores before the reads
            __syncthreads();
            const int64_t nr = r0 + NT / 64 < pr.q.R ? NT / 64 : pr.q.R - r0;
            const int64_t gpr = pr.q.K / 32;
            for (int64_t g = tid; g < nr * gpr; g += NT) quant_group_mxfp4(pr.q, r0 * gpr + g);
        }
    }
}

}  // namespace moe
