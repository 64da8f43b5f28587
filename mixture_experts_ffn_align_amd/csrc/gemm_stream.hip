// Grouped expert GEMMs of the fused MoE forward, weight-streaming variant.
//
// Stage 1 (gemm1 + act): for one sorted block of BM rows, all routed to
// expert e, the rows of x they came from (t = a / k) times gate_e^T and
// up_e^T, then h = SiLU(g) * u (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs
// for Qwen3.5-397B", Details: ActivationType.Silu). gate and up are addressed
// through their own expert and row strides, so views into one packed
// w13 [E, 2I, H] are read in place (Liger-Kernel PR #1377, Problems: each
// expert's first weight tile must come from the real expert stride, not from
// I / TileN).
// Stage 2 (gemm2): h rows times w2_e^T, each fp32 result row written to its
// flat assignment index a = t*k + j, ready for the slot-ordered combine. h
// itself is stored by flat assignment index too, so the two stages may use
// differently padded sorted layouts.
//
// Work split. A workgroup is four wave64s. Each wave owns 4 MFMA column
// blocks of 16 (stage 1: 32 gate + 32 up rows -> 32 h columns; stage 2: 64
// output columns) for all BM rows; WK waves split K and reduce through LDS
// in a fixed order. Both operands are K-contiguous, which is exactly the
// per-lane layout of v_mfma_f32_16x16x32_bf16 / v_mfma_scale_f32_16x16x128
// (lane l: row l % 16, a run of consecutive k chosen by l / 16):
//  * weights (B) are read by exactly one wave, so every lane loads its
//    16-byte operand straight from HBM into registers, the next U steps
//    always in flight while the current ones multiply;
//  * token rows (A) are shared by the waves that split N, so they are staged
//    once per workgroup in LDS, already in MFMA fragment order: lane l of
//    the loading wave writes offset 16*l of a 1 KB fragment, and a consuming
//    wave reads the same offset back with one ds_read_b128. Chunks of cs
//    steps are double buffered: the next chunk is loaded into a few VGPRs
//    at the start of a chunk and written to the idle buffer at its end, with
//    one workgroup barrier per chunk that waits on LDS only, never on the
//    weight loads in flight.
//
// In MXFP4 mode one lane's 32 e2m1 codes are exactly one scale block, so the
// per-1x32 e8m0 scales feed the block-scaled MFMA directly, and the stage 1
// epilogue quantises h per 32 columns in registers (max over 16 lanes).
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

template <int MODE>
struct Frag;
template <>
struct Frag<0> {          // bf16: 8 values per lane per step
    bf16x8_t v;
};
template <>
struct Frag<1> {          // fp4: 32 codes (16 bytes) per lane per step
    i32x4_t v;
};

// Occupancy target per SIMD: the weight stream needs as many waves in flight
// as the register file allows, so the allocation is capped (bf16: 4 waves
// for 16 rows, 3 for 32, 2 for 64 and 128; MXFP4, whose ring also carries
// scale windows: 3 for 16 rows, else 2).
template <int MODE, int BM, int WK, int NB>
constexpr int waves_per_simd() {
    if (MODE == 1) return BM <= 16 ? 3 : 2;
    return NB == 2 ? (BM <= 32 ? 4 : 3) : (BM <= 16 ? (WK == 1 ? 4 : 3) : (BM <= 32 ? 3 : 2));
}

template <int MODE, int STAGE, int BM, int WK, int U, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_simd<MODE, BM, WK, NB>(), 8)))
void gemm_stream(GemmParams p) {
    static_assert(NB == 2 || NB == 4, "a wave owns 2 or 4 column blocks of 16");
    static_assert(MODE == 0 || STAGE == 2 || NB == 4, "MXFP4 h quantisation needs 32 h columns per wave");
    constexpr int MB = BM / 16;
    constexpr int WN = 4 / WK;
    constexpr int KSTEP = MODE == 0 ? 32 : 128;
    constexpr int WCOLS = STAGE == 1 ? NB * 8 : NB * 16;
    constexpr int TILE_N = WN * WCOLS;
    // 1 KB A fragments per LDS buffer: room for a chunk of at least 2U steps
    // (MXFP4 with a 4-step ring stages its weight scales in LDS and keeps
    // 8-fragment A chunks so that three workgroups still fit a CU)
    constexpr bool SC_LDS = MODE == 1 && U == 4;
    constexpr int FRAGS_MIN = SC_LDS ? 8 : 16;
    constexpr int FRAGS = (U * WK * MB > FRAGS_MIN) ? U * WK * MB : FRAGS_MIN;
    static_assert(FRAGS % 4 == 0 && 2 * FRAGS <= 64, "A staging must fit 64 KB of LDS");
    constexpr int RED_FLOATS = 4 * MB * NB * 4 * 64;
    constexpr int LDS_FLOATS = (WK > 1 && RED_FLOATS > 2 * FRAGS * 256) ? RED_FLOATS : 2 * FRAGS * 256;
    constexpr int AREGS = FRAGS / 4;      // fragments one wave stages per chunk (at most)
    __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
    // MXFP4 weight scales of the wave's 64 rows over its whole K share
    // (row-major, K/32 bytes per row, for K up to 4096), loaded once
    constexpr int SC_ROW_MAX = 128 / WK;
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[SC_LDS ? 4 * 64 * SC_ROW_MAX : 16];

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wn = w / WK, wk = w % WK;
    const int r16 = lane & 15, kg = lane >> 4;

    // ---- tile mapping: ((n-group, m-block), n-tile in group). Consecutive
    // workgroups go to different XCDs, which spreads the weight stream of
    // neighbouring tiles over all of them; pinning a contiguous tile range to
    // one XCD measured slower for this stream.
    const int n_tiles = p.N / TILE_N;
    const uint32_t L = blockIdx.x;
    const int G = p.n_tile_groups;
    const int ji = (int)(L % (uint32_t)G);
    const uint32_t rest = L / (uint32_t)G;
    const int mb = (int)(rest % (uint32_t)p.max_mblocks);
    const int jg = (int)(rest / (uint32_t)p.max_mblocks);
    const int nt = jg * G + ji;
    if (nt >= n_tiles) return;
    const int n_blocks = *p.n_padded / BM;
    if (mb >= n_blocks) return;
    const int e = p.block_expert[mb];
    const int row0 = mb * BM;
    const int n0 = nt * TILE_N + wn * WCOLS;

    // ---- operand row addresses (per lane)
    const char* a_ptr[MB];
    const uint8_t* a_sc[MB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
        // stage 1 gathers the token row t = a / k; stage 2 the h row of the
        // flat assignment a; a padding row re-reads row 0
        const int a = p.sorted[row0 + mi * 16 + r16];
        const int64_t arow = a < p.A ? (STAGE == 1 ? (int64_t)((unsigned)a / (unsigned)p.k) : (int64_t)a) : 0;
        if (MODE == 0) {
            a_ptr[mi] = reinterpret_cast<const char*>(p.a) + arow * p.a_row * 2;
            a_sc[mi] = nullptr;
        } else {
            a_ptr[mi] = reinterpret_cast<const char*>(p.a) + arow * p.a_row;
            a_sc[mi] = p.a_sc + arow * p.a_sc_row;
        }
    }
    const char* b_ptr[NB];
    const uint8_t* b_sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const bool second = STAGE == 1 && nb >= NB / 2;
        const int wrow = STAGE == 1 ? n0 + (nb % (NB / 2)) * 16 + r16 : n0 + nb * 16 + r16;
        const char* base = reinterpret_cast<const char*>(second ? p.b1 : p.b0);
        const int64_t se = second ? p.b1_e : p.b0_e;
        const int64_t sr = second ? p.b1_r : p.b0_r;
        if (MODE == 0) {
            b_ptr[nb] = base + ((int64_t)e * se + (int64_t)wrow * sr) * 2;
            b_sc[nb] = nullptr;
        } else {
            b_ptr[nb] = base + (int64_t)e * se + (int64_t)wrow * sr;
            const uint8_t* sb = second ? p.b1_sc : p.b0_sc;
            const int64_t sse = second ? p.b1sc_e : p.b0sc_e;
            const int64_t ssr = second ? p.b1sc_r : p.b0sc_r;
            b_sc[nb] = sb + (int64_t)e * sse + (int64_t)wrow * ssr;
        }
    }

    // ---- K loop
    const int kw = p.K / WK;
    const int steps = kw / KSTEP;                 // steps per wave; the host keeps it a multiple of 2U
    // byte offset of a lane's operand run for step s of K share q
    auto koff = [&](int q, int s) -> int64_t {
        const int k = q * kw + s * KSTEP;
        return MODE == 0 ? (int64_t)(k + kg * 8) * 2 : (int64_t)(k / 2 + kg * 16);
    };
    // A chunks of cs steps: a multiple of U that divides steps, at most
    // FRAGS fragments per buffer
    int cs = FRAGS / (WK * MB);
    cs = cs < steps ? cs : steps;
    cs = cs < U ? U : cs - cs % U;
    while (steps % cs != 0) cs -= U;
    const int nac = steps / cs;
    const int nfrag = WK * MB * cs;              // fragments per chunk (<= FRAGS)
    char* const lds_bytes = reinterpret_cast<char*>(lds);
    // fragment f = (q * MB + mi) * cs + st of buffer b sits at (b * FRAGS + f) KB;
    // wave w stages fragments f = w, w + 4, ...
    i32x4_t areg[AREGS];
    // Both are branch-free (slots past nfrag load a valid fragment again and
    // fill unused LDS), so the compiler's wait counts stay exact.
    auto load_A = [&](int ac) {
#pragma unroll
        for (int i = 0; i < AREGS; ++i) {
            int f = w + 4 * i;
            f = f < nfrag ? f : nfrag - 1;
            const int st = f % cs, qm = f / cs;
            const int q = qm / MB, mi = qm % MB;
            const char* src = a_ptr[0];
#pragma unroll
            for (int m = 1; m < MB; ++m) src = m == mi ? a_ptr[m] : src;
            areg[i] = *reinterpret_cast<const i32x4_t*>(src + koff(q, ac * cs + st));
        }
    };
    auto store_A = [&](int b) {
#pragma unroll
        for (int i = 0; i < AREGS; ++i)
            *reinterpret_cast<i32x4_t*>(lds_bytes + ((size_t)(b * FRAGS + w + 4 * i) << 10) + lane * 16) = areg[i];
    };

    // Weights: a ring of U step-slots per wave. Slot u holds step s+u; right
    // after its MFMAs consume it, it is refilled with step s+u+U, so U-1
    // steps of weight loads are always in flight.
    Frag<MODE> fb[U][NB];
    // MXFP4 scales: per ring round, one window of 4*U bytes per row (all four
    // k-groups of the U steps) in one load per row; byte 4u+kg of the window is
    // this lane's scale for step u. The next round's window loads with the
    // round's first refill.
    // After a window lands, byte u of the packed word is this lane's scale for
    // step u of the round.
    uint32_t bsc[NB], asc[MB], bsc_n[NB][U], asc_n[MB][U];
    f32x4_t acc[MB][NB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mi][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load_B = [&](int slot, int st) {
        st = st < steps ? st : steps - 1;       // past the end: re-read the last step (L2 hit)
        const int64_t off = koff(wk, st);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            using V = decltype(fb[slot][nb].v);
            fb[slot][nb].v = *reinterpret_cast<const V*>(b_ptr[nb] + off);
        }
    };
    using SW = typename std::conditional<U == 4, i32x4_t, int __attribute__((ext_vector_type(2)))>::type;
    auto pack_scales = [&]() {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint32_t v = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) v |= ((bsc_n[nb][u] >> (8 * kg)) & 0xffu) << (8 * u);
            bsc[nb] = v;
        }
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            uint32_t v = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) v |= ((asc_n[mi][u] >> (8 * kg)) & 0xffu) << (8 * u);
            asc[mi] = v;
        }
    };
    // The weight scales of a row are one contiguous run of K/32 bytes; read
    // window by window from global memory, a run is fetched again for every
    // window once the weight stream has evicted it. Where the run fits
    // (K <= 4096), each wave loads its 64 rows' runs once, straight into
    // LDS, and the windows are read from there.
    // (the host gives MXFP4 a 4-step ring only where the run of every row
    // fits SC_ROW_MAX and lpr divides 64)
    const int sc_bpr = kw / 32;                          // scale bytes per row of the K share
    uint8_t* const sc_wave = sc_lds + w * 64 * SC_ROW_MAX;
    if constexpr (SC_LDS) {
        // instruction i: rows i*rpi .. +rpi, lpr lanes x 16 bytes per row;
        // LDS block i (1 KB) is rows i*rpi .. in row-major order
        const int lpr = sc_bpr / 16, rpi = 64 / lpr;
        const int rr = lane / lpr, cc = lane % lpr;
        for (int i = 0; i < lpr; ++i) {
            const int row = i * rpi + rr;                 // 0 .. 63
            const int nb = row / 16, r = row % 16;
            const bool second = STAGE == 1 && nb >= NB / 2;
            const int wrow = STAGE == 1 ? n0 + (nb % (NB / 2)) * 16 + r : n0 + nb * 16 + r;
            const uint8_t* src = (second ? p.b1_sc : p.b0_sc) + (int64_t)e * (second ? p.b1sc_e : p.b0sc_e) +
                                 (int64_t)wrow * (second ? p.b1sc_r : p.b0sc_r) + wk * sc_bpr + cc * 16;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                             (__attribute__((address_space(3))) void*)(sc_wave + i * 1024), 16, 0,
                                             0);
        }
    }
    auto load_scales = [&](uint32_t (&bdst)[NB][U], uint32_t (&adst)[MB][U], int s0) {
        if constexpr (MODE == 1) {
            s0 = s0 < steps - U ? s0 : steps - U;
            const int kb0 = (wk * kw + s0 * KSTEP) / 32;     // a multiple of 4*U
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                SW v;
                if constexpr (SC_LDS)
                    v = *reinterpret_cast<const SW*>(sc_wave + (nb * 16 + r16) * sc_bpr + s0 * (KSTEP / 32));
                else
                    v = *reinterpret_cast<const SW*>(b_sc[nb] + kb0);
#pragma unroll
                for (int u = 0; u < U; ++u) bdst[nb][u] = (uint32_t)v[u];
            }
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) {
                const SW v = *reinterpret_cast<const SW*>(a_sc[mi] + kb0);
#pragma unroll
                for (int u = 0; u < U; ++u) adst[mi][u] = (uint32_t)v[u];
            }
        }
    };
    auto compute = [&](int slot, const char* abuf, int sl) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const char* src = abuf + (size_t)(((wk * MB + mi) * cs + sl) << 10) + lane * 16;
            const i32x4_t araw = *reinterpret_cast<const i32x4_t*>(src);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (MODE == 0) {
                    acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, araw), fb[slot][nb].v, acc[mi][nb], 0, 0, 0);
                } else {
                    const i32x4_t bv = fb[slot][nb].v;
                    const i32x8_t a8 = {araw[0], araw[1], araw[2], araw[3], 0, 0, 0, 0};
                    const i32x8_t b8 = {bv[0], bv[1], bv[2], bv[3], 0, 0, 0, 0};
                    acc[mi][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a8, b8, acc[mi][nb], 4, 4, 0, (int)(asc[mi] >> (8 * slot)), 0,
                        (int)(bsc[nb] >> (8 * slot)));
                }
            }
        }
    };
    // U steps starting at s0 (a multiple of U) of A chunk ac; every slot is
    // refilled right after use, unconditionally, so wait counts stay exact
    auto ring = [&](const char* abuf, int ac, int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            compute(u, abuf, s0 + u - ac * cs);
            __builtin_amdgcn_sched_barrier(0);
            load_B(u, s0 + u + U);
            if (u == 0) load_scales(bsc_n, asc_n, s0 + U);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MODE == 1) pack_scales();
    };
    // LDS-only workgroup barrier: waits for this wave's LDS writes, not for
    // the weight loads in flight
    auto lds_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int u = 0; u < U; ++u) load_B(u, u);
    load_scales(bsc_n, asc_n, 0);
    if constexpr (MODE == 1) pack_scales();
    load_A(0);
    store_A(0);
    for (int ac = 0; ac < nac; ++ac) {
        lds_barrier();                             // chunk ac visible; buffer (ac+1)&1 idle
        const char* abuf = lds_bytes + ((size_t)((ac & 1) * FRAGS) << 10);
        load_A(ac + 1 < nac ? ac + 1 : ac);        // next chunk into registers
        __builtin_amdgcn_sched_barrier(0);
        // the first U steps are peeled so that the next chunk goes to LDS at a
        // point where its loads are known to be older than the weight loads in
        // flight (no drain of the weight stream)
        ring(abuf, ac, ac * cs);
        store_A((ac + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int s0 = ac * cs + U; s0 < (ac + 1) * cs; s0 += U) ring(abuf, ac, s0);
    }

    // ---- split-K reduction through LDS (fixed order wk = 0..WK-1); the
    // buffer reuses the A chunks, so every wave must be done reading them
    float* red = lds;
    if constexpr (WK > 1) {
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[(((w * MB + mi) * NB + nb) * 4 + i) * 64 + lane] = acc[mi][nb][i];
        __syncthreads();
    }
    auto tile = [&](int mi, int nb) -> f32x4_t {
        if constexpr (WK == 1) {
            return acc[mi][nb];
        } else {
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < WK; ++q) {
                const int src = wn * WK + q;
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] += red[(((src * MB + mi) * NB + nb) * 4 + i) * 64 + lane];
            }
            return s;
        }
    };

    // ---- epilogues
    if constexpr (STAGE == 1 && MODE == 0) {
        uint16_t* h = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int unit = 0; unit < MB * (NB / 2); ++unit) {
            if (unit % WK != wk) continue;
            const int mi = unit / (NB / 2), np = unit % (NB / 2);
            const f32x4_t g = tile(mi, np), u = tile(mi, np + NB / 2);
            const int col = n0 + np * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = p.sorted[row0 + mi * 16 + kg * 4 + i];   // h rows by flat assignment
                if (a < p.A) h[(int64_t)a * p.N + col] = f32_to_bf16_bits(silu_mul(g[i], u[i]));
            }
        }
    } else if constexpr (STAGE == 1 && MODE == 1) {
        uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            if (mi % WK != wk) continue;
            const f32x4_t g0 = tile(mi, 0), g1 = tile(mi, 1), u0 = tile(mi, 2), u1 = tile(mi, 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float h0 = silu_mul(g0[i], u0[i]);
                const float h1 = silu_mul(g1[i], u1[i]);
                const uint32_t b0 = __float_as_uint(h0), b1 = __float_as_uint(h1);
                uint32_t amax = max(b0 & 0x7fffffffu, b1 & 0x7fffffffu);
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
                const int s = group_exponent(amax);
                const E2m1Thresholds th = e2m1_thresholds(s);
                const uint32_t c0 = e2m1_code(b0, th), c1 = e2m1_code(b1, th);
                const uint32_t o0 = (uint32_t)__shfl_xor((int)c0, 1), o1 = (uint32_t)__shfl_xor((int)c1, 1);
                const int a = p.sorted[row0 + mi * 16 + kg * 4 + i];   // h rows by flat assignment
                if (a >= p.A) continue;
                uint8_t* rp = hq + (int64_t)a * (p.N / 2);
                if ((r16 & 1) == 0) {
                    rp[(n0 + r16) / 2] = (uint8_t)(c0 | (o0 << 4));
                    rp[(n0 + 16 + r16) / 2] = (uint8_t)(c1 | (o1 << 4));
                }
                if (r16 == 0) p.out_sc[(int64_t)a * (p.N / 32) + n0 / 32] = (uint8_t)(s + 127);
            }
        }
    } else {
        // y rows in bf16 (RNE)
        uint16_t* y16 = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int unit = 0; unit < MB * NB; ++unit) {
            if (unit % WK != wk) continue;
            const int mi = unit / NB, nb = unit % NB;
            const f32x4_t t = tile(mi, nb);
            const int col = n0 + nb * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = p.sorted[row0 + mi * 16 + kg * 4 + i];
                if (a >= p.A) continue;
                y16[(int64_t)a * p.out_row + col] = f32_to_bf16_bits(t[i]);
            }
        }
    }
}

// MXFP4 gemm2 when a wave's whole K is one ring round (K = 4 steps of 128,
// the TP2 shard's I = 512): a workgroup takes NT consecutive 256-column
// tiles of one row block instead of one. The h rows (the A operand, all of K)
// are staged in LDS once and serve every tile; each wave DMA-loads the scale
// rows of all its tiles once; the weight ring runs on across tiles (slot u
// of tile j + 1 loads right after slot u of tile j is multiplied), so tile
// j's epilogue and tile j + 1's first MFMAs overlap its loads. The weight
// fragment is the MFMA's first operand: a lane's accumulator holds 4
// consecutive output columns of one row and stores them as one 8-byte write.
template <int BM, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void gemm_stream_nt(GemmParams p) {
    constexpr int MB = BM / 16, NB = 4, U = 4;
    constexpr int TILE_N = 4 * NB * 16;                       // 256 columns, 64 per wave
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[MB * U * 1024];    // fragment (mi, u): 1 KB
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[4 * NT * 1024];   // wave, tile: 64 rows x 16 B
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;

    // workgroups of one row block are consecutive, NT tiles each
    const int n_tiles = p.N / TILE_N;
    const int n_groups = (n_tiles + NT - 1) / NT;
    const int tg = (int)(blockIdx.x % (uint32_t)n_groups);
    const int mb = (int)(blockIdx.x / (uint32_t)n_groups);
    if (mb >= p.max_mblocks) return;
    const int n_blocks = *p.n_padded / BM;
    if (mb >= n_blocks) return;
    const int e = p.block_expert[mb];
    const int row0 = mb * BM;
    const int nt0 = tg * NT;
    const int ntn = min(NT, n_tiles - nt0);                   // tiles of this workgroup, >= 1
    auto col0 = [&](int j) { return (nt0 + j) * TILE_N + w * (NB * 16); };   // the wave's first column

    // weight scale rows of every tile: one 16-byte run (K/32 bytes) per row,
    // lane l of the wave's DMA for tile j fetches row col0(j) + l
    for (int j = 0; j < ntn; ++j)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(p.b0_sc + (int64_t)e * p.b0sc_e + (int64_t)(col0(j) + lane) * p.b0sc_r),
            (__attribute__((address_space(3))) void*)(sc_lds + (w * NT + j) * 1024), 16, 0, 0);

    // h rows of the block: flat assignment a (a padding row re-reads row 0)
    int arow[MB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
        const int a = p.sorted[row0 + mi * 16 + r16];
        arow[mi] = a;
    }
    // A fragments: wave w stages (mi, u) = f for f = w, w + 4, ...
    i32x4_t areg[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int f = w + 4 * i, mi = f / U, u = f % U;
        const int64_t r = arow[mi] < p.A ? arow[mi] : 0;
        areg[i] = *reinterpret_cast<const i32x4_t*>(reinterpret_cast<const char*>(p.a) + r * p.a_row + u * 64 +
                                                    kg * 16);
    }
    // A scales: the whole K of a row is one 16-byte window; byte 4u + kg is
    // this lane's scale for step u, packed so that byte u is step u
    uint32_t asc[MB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
        const int64_t r = arow[mi] < p.A ? arow[mi] : 0;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(p.a_sc + r * p.a_sc_row);
        uint32_t pk = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) pk |= (((uint32_t)v[u] >> (8 * kg)) & 0xffu) << (8 * u);
        asc[mi] = pk;
    }
    // weight ring: slot u holds step u of the current tile
    const char* bbase = reinterpret_cast<const char*>(p.b0) + (int64_t)e * p.b0_e;
    i32x4_t fb[U][NB];
    auto load_B = [&](int u, int j) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            fb[u][nb] = *reinterpret_cast<const i32x4_t*>(bbase + (int64_t)(col0(j) + nb * 16 + r16) * p.b0_r +
                                                          u * 64 + kg * 16);
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_B(u, 0);
#pragma unroll
    for (int i = 0; i < MB; ++i)
        *reinterpret_cast<i32x4_t*>(a_lds + (w + 4 * i) * 1024 + lane * 16) = areg[i];
    __syncthreads();

    uint16_t* y = reinterpret_cast<uint16_t*>(p.out);
    // the accumulators are carried around the tile loop (zeroed after each
    // epilogue), so every MFMA accumulates in place
    f32x4_t acc[MB][NB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float z;
            __asm__("v_mov_b32 %0, 0" : "=v"(z));
            acc[mi][nb] = f32x4_t{z, z, z, z};
        }
#pragma unroll 1
    for (int j = 0; j < ntn; ++j) {
        // this tile's weight scales, packed like the A scales
        uint32_t bsc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const i32x4_t v = *reinterpret_cast<const i32x4_t*>(sc_lds + (w * NT + j) * 1024 + (nb * 16 + r16) * 16);
            uint32_t pk = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) pk |= (((uint32_t)v[u] >> (8 * kg)) & 0xffu) << (8 * u);
            bsc[nb] = pk;
        }
        const int jn = j + 1 < ntn ? j + 1 : j;               // past the last tile: re-read it (L2 hit)
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) {
                const i32x4_t af = *reinterpret_cast<const i32x4_t*>(a_lds + (mi * U + u) * 1024 + lane * 16);
                const i32x8_t a8 = {af[0], af[1], af[2], af[3], 0, 0, 0, 0};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const i32x8_t b8 = {fb[u][nb][0], fb[u][nb][1], fb[u][nb][2], fb[u][nb][3], 0, 0, 0, 0};
                    acc[mi][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        b8, a8, acc[mi][nb], 4, 4, 0, (int)(bsc[nb] >> (8 * u)), 0, (int)(asc[mi] >> (8 * u)));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            load_B(u, jn);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The MFMAs read operands from every lane, so they must run with all
        // lanes on: pin the results here, before the per-row branch below,
        // which the compiler would otherwise sink them into.
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) __asm__ volatile("" : "+v"(acc[mi][nb]));
        // y rows by flat assignment (bf16, RNE): lane holds columns 4 kg ..
        // +3 of column block nb for row r16
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            if (arow[mi] >= p.A) continue;
            uint16_t* yr = y + (int64_t)arow[mi] * p.out_row + col0(j) + kg * 4;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                const u32x2_t pk = {
                    bf16x2_bits(acc[mi][nb][0], acc[mi][nb][1]),
                    bf16x2_bits(acc[mi][nb][2], acc[mi][nb][3])};
                __builtin_nontemporal_store(pk, reinterpret_cast<u32x2_t*>(yr + nb * 16));
            }
        }
        // zeroed through registers the compiler cannot see as constants, so
        // that the first MFMA of the next tile accumulates in place too
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float z;
                __asm__("v_mov_b32 %0, 0" : "=v"(z));
                acc[mi][nb] = f32x4_t{z, z, z, z};
            }
    }
}

typedef void (*GemmFn)(GemmParams);

template <int MODE, int STAGE, int BM, int WK, int U, int NB = 4>
constexpr GemmFn pick() {
    return gemm_stream<MODE, STAGE, BM, WK, U, NB>;
}

template <int MODE, int STAGE, int U>
GemmFn table(int bm, int wk) {
#define MOE_CASE(B, W) \
    if (bm == B && wk == W) return pick<MODE, STAGE, B, W, U>();
    MOE_CASE(16, 1) MOE_CASE(16, 2) MOE_CASE(16, 4)
    MOE_CASE(32, 1) MOE_CASE(32, 2) MOE_CASE(32, 4)
    MOE_CASE(64, 1) MOE_CASE(64, 2)
#undef MOE_CASE
    return nullptr;
}

template <int MODE, int STAGE>
GemmFn table_u(int bm, int wk, int u, int nb) {
    if constexpr (MODE == 0) {
        // narrow waves (2 column blocks, a ring of 8) for the weight stream
        if (nb == 2) {
            if (wk != 1 || u != 8) return nullptr;
            if (bm == 32) return pick<MODE, STAGE, 32, 1, 8, 2>();
            if (bm == 64) return pick<MODE, STAGE, 64, 1, 8, 2>();
            return nullptr;
        }
    }
    if (nb != 4) return nullptr;
    if (bm == 128 && wk == 1) return u == 2 ? pick<MODE, STAGE, 128, 1, 2>() : nullptr;
    if (u == 4) return table<MODE, STAGE, 4>(bm, wk);
    if constexpr (MODE == 1) {
        if (u == 2) return table<MODE, STAGE, 2>(bm, wk);
    }
    return nullptr;
}

// The weight ring holds 4 steps (bf16: 32 k each; MXFP4: 128 k each, where a
// wave's share of K allows it, else 2); with 128 rows the accumulators leave
// room for 2; narrow bf16 waves hold 8.
GemmFn lookup(const GemmKernelId& id) {
    if (id.nt != 1) {
        if (id.mode != 1 || id.stage != 2 || id.wk != 1 || id.u != 4 || id.nb != 4) return nullptr;
#define MOE_NT(B, T) \
    if (id.bm == B && id.nt == T) return gemm_stream_nt<B, T>;
        MOE_NT(16, 2) MOE_NT(16, 4) MOE_NT(16, 8) MOE_NT(32, 2) MOE_NT(32, 4) MOE_NT(32, 8)
        MOE_NT(64, 2) MOE_NT(64, 4) MOE_NT(64, 8)
#undef MOE_NT
        return nullptr;
    }
    if (id.mode == 0)
        return id.stage == 1 ? table_u<0, 1>(id.bm, id.wk, id.u, id.nb) : table_u<0, 2>(id.bm, id.wk, id.u, id.nb);
    if (id.mode == 1)
        return id.stage == 1 ? table_u<1, 1>(id.bm, id.wk, id.u, id.nb) : table_u<1, 2>(id.bm, id.wk, id.u, id.nb);
    return nullptr;
}

}  // namespace

int gemm_ring_steps(int mode, int bm, int nb, int wk, int64_t k_per_wave) {
    if (mode == 0 && nb == 2) return 8;
    if (bm >= 128) return 2;
    if (mode == 0) return 4;
    // a 4-step MXFP4 ring stages the share's weight scales in LDS: each row's
    // run of k_per_wave / 32 bytes must fit the 128 / wk bytes per row the
    // kernel reserves, and goes in 16-byte pieces, k_per_wave / 512 lanes per
    // row, so the wave's 64 lanes must cover whole rows
    const int64_t lanes_per_row = k_per_wave / 512;
    return k_per_wave % 512 == 0 && k_per_wave / 32 <= 128 / wk && 64 % lanes_per_row == 0 ? 4 : 2;
}

int gemm_k_granule(const GemmKernelId& id) {
    return id.mode == 0 ? 32 * (id.nb == 2 ? 8 : 4) : 128 * 2;
}

int gemm_tile_n(const GemmKernelId& id) {
    const int wn = 4 / id.wk;
    return wn * (id.stage == 1 ? id.nb * 8 : id.nb * 16);
}

bool gemm_supported(const GemmKernelId& id) { return lookup(id) != nullptr; }

namespace {

// MXFP4 gemm2 and combine in one pass, for a few tokens: one workgroup per
// token t and 16 output columns n0 .. n0 + 15, of W = min(ceil(k / S), 16)
// waves. Wave w takes slots j = w, w + W, ... (S of them per round), issuing
// the loads of a round before it waits on any; for a slot it multiplies the
// 16 w2 rows of the slot's expert by the slot's h row with the same MFMA
// sequence as the weight streams (weights as the first operand, K = 512 in
// four 128-steps from zero) and leaves y rounded to bf16 in LDS. Then 16 lanes of wave 0
// add w_tj * y over j in slot order with fmaf, exactly as the separate
// combine does; so the output is bit-identical to gemm2 followed by the
// combine, without y in memory.
constexpr int kG2cMaxK = 64;

// LOOP: k > S * W, the slots in rounds of S * W (a loop makes the compiler's
// waits cover earlier loads, so the common single round has no loop)
template <int S, bool LOOP>
__global__ __launch_bounds__(1024) void gemm2_combine_kernel(Gemm2CombineParams q) {
    const GemmParams& p = q.g;
    const CombineParams& c = q.c;
    constexpr int U = 4;
    __shared__ float ys[kG2cMaxK][16];
    __shared__ float wts[kG2cMaxK];
    __shared__ int eid[kG2cMaxK];                    // local expert, or -1
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int ncb = p.N / 16;
    const int64_t t = blockIdx.x / (uint32_t)ncb;
    const int n0 = (int)(blockIdx.x % (uint32_t)ncb) * 16;
    if (t >= c.T) return;
    // the token's ids and weights once, so that no wave waits on them
    // between its weight loads
    if (threadIdx.x < c.k) {
        const int j = threadIdx.x;
        const int64_t e = (int64_t)c.ids[t * c.is_t + (int64_t)j * c.is_j] - c.e_off;
        eid[j] = e >= 0 && e < c.E ? (int)e : -1;
        wts[j] = c.w[t * c.ws_t + (int64_t)j * c.ws_j];
    }
    __syncthreads();
    auto round = [&](const int base) {
        bool ok[S];
        i32x4_t fb[S][U], fa[S][U], vb[S], va[S];
#pragma unroll
        for (int h = 0; h < S; ++h) {
            const int j = base + w + h * W;
            const int64_t e = j < c.k ? __builtin_amdgcn_readfirstlane(eid[j]) : -1;
            ok[h] = e >= 0;
            if (ok[h]) {
                const int64_t a = t * c.k + j;
                const char* wr = reinterpret_cast<const char*>(p.b0) + e * p.b0_e + (int64_t)(n0 + r16) * p.b0_r;
                const char* hr = reinterpret_cast<const char*>(p.a) + a * p.a_row;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    fb[h][u] = *reinterpret_cast<const i32x4_t*>(wr + u * 64 + kg * 16);
                    fa[h][u] = *reinterpret_cast<const i32x4_t*>(hr + u * 64 + kg * 16);
                }
                vb[h] = *reinterpret_cast<const i32x4_t*>(p.b0_sc + e * p.b0sc_e + (int64_t)(n0 + r16) * p.b0sc_r);
                va[h] = *reinterpret_cast<const i32x4_t*>(p.a_sc + a * p.a_sc_row);
            }
        }
#pragma unroll
        for (int h = 0; h < S; ++h) {
            if (!ok[h]) continue;
            // byte 4u + kg of a scale window is this lane's for step u
            f32x4_t acc;
            {
                float z;
                __asm__("v_mov_b32 %0, 0" : "=v"(z));
                acc = f32x4_t{z, z, z, z};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const i32x8_t b8 = {fb[h][u][0], fb[h][u][1], fb[h][u][2], fb[h][u][3], 0, 0, 0, 0};
                const i32x8_t a8 = {fa[h][u][0], fa[h][u][1], fa[h][u][2], fa[h][u][3], 0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc, 4, 4, 0,
                                                                        (int)((uint32_t)vb[h][u] >> (8 * kg)), 0,
                                                                        (int)((uint32_t)va[h][u] >> (8 * kg)));
            }
            __asm__ volatile("" : "+v"(acc));
            // lane (r16, kg) holds columns 4 kg + i; every r16 the same
            if (r16 == 0) {
                const int j = base + w + h * W;
#pragma unroll
                for (int i = 0; i < 4; ++i) ys[j][4 * kg + i] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
            }
        }
    };
    if constexpr (LOOP) {
        for (int base = 0; base < c.k; base += S * W) round(base);
    } else {
        round(0);
    }
    __syncthreads();
    if (w != 0 || lane >= 16) return;
    float out_acc = 0.f;
    for (int j = 0; j < c.k; ++j)
        if (eid[j] >= 0) out_acc = __builtin_fmaf(wts[j], ys[j][lane], out_acc);
    c.out[t * c.os_t + (int64_t)(n0 + lane) * c.os_h] = (uint16_t)f32_to_bf16_bits(out_acc);
}

}  // namespace

namespace {

// MXFP4 gemm1 for a few tokens, without the align. Workgroup (slot a, h
// columns c0 .. c0 + 31): K = H is split in quarters, and each MFMA block
// chains over its quarter in ascending 128-steps from zero (weights first:
// gate rows c0 .. c0 + 31 in blocks 0, 1, up rows in blocks 2, 3); the
// partial sums meet in LDS and are added in quarter order ((p0 + p1) + p2) +
// p3, exactly as the register weight stream with a 4-way K split does. The
// workgroup first quantises its token's activation row into LDS with the
// quantisation kernel's arithmetic. So the h codes and scales are
// bit-identical to the aligned path's with that split. Every lane
// multiplies the same token row, so the 16 MFMA columns hold copies of one
// result.
//
// With one to a few tokens the weight stream is all the traffic and each
// wave has little else to do, so a wave issues the loads of up to 8 steps
// (16 bytes per lane, step and block, plus one 16-byte scale window per 4
// steps and block) before it waits on any: with two blocks per wave, 16 KB
// in flight per wave.
constexpr int kSmallMaxH = 8192;
constexpr int kSmallChunk = 8;
constexpr int kSmallBPW = 2;                    // measured: 2 beats 4 and 1 at T = 1-16

// STEPS: 128-steps per wave, H / 512 (a compile-time count keeps the load
// waits exact). BPW: MFMA blocks per wave (4, 2 or 1); the workgroup has
// 4 x 4 / BPW waves, wave w taking K quarter w % 4 of blocks
// (w / 4) BPW .. + BPW - 1. Every element's sum is the same for any BPW.
template <int STEPS, int BPW>
__global__ __launch_bounds__(256 * (4 / BPW)) void gemm1_small_kernel(Gemm1SmallParams p) {
    constexpr int NT = 256 * (4 / BPW);
    __shared__ uint4 xcode[kSmallMaxH / 32];         // the row's e2m1 codes, 32 per entry
    __shared__ uint8_t xscale[kSmallMaxH / 32];
    __shared__ float red[4][4][4][64];
    static_assert(sizeof(red) >= kSmallMaxH * 2, "the reduction buffer holds a bf16 row");
    __shared__ float rsc;                            // the row's RMSNorm scale
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qk = w & 3, b0 = (w >> 2) * BPW;
    const int r16 = lane & 15, kg = lane >> 4;
    const int ncb = p.I / 32;
    const int a = (int)(blockIdx.x / (uint32_t)ncb);
    const int c0 = (int)(blockIdx.x % (uint32_t)ncb) * 32;
    if (a >= p.A) return;
    const int64_t t = a / p.k, j = a % p.k;
    const int64_t e = (int64_t)p.ids[t * p.is_t + j * p.is_j] - p.e_off;
    if (e < 0 || e >= p.E) return;                   // the same for the whole workgroup
    const int kq = p.H / 4;                          // this wave's quarter of K
    const int kbase = qk * kq;
    const uint8_t* wr[BPW];
    const uint8_t* sr[BPW];
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
        const int b = b0 + bl;
        const int row = c0 + 16 * (b & 1) + r16;
        wr[bl] = b < 2 ? p.gate + e * p.g_e + (int64_t)row * p.g_r : p.up + e * p.u_e + (int64_t)row * p.u_r;
        sr[bl] = b < 2 ? p.gate_sc + e * p.gs_e + (int64_t)row * p.gs_r
                       : p.up_sc + e * p.us_e + (int64_t)row * p.us_r;
    }
    f32x4_t acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        float z;
        __asm__("v_mov_b32 %0, 0" : "=v"(z));
        acc[b] = f32x4_t{z, z, z, z};
    }
    // the activation row is quantised 8 values per thread and pass (groups
    // of 32 are 4 neighbouring lanes); a contiguous row is loaded before the
    // weights so that its wait does not cover them
    const uint16_t* xr = p.x + t * p.xs_t;
    const bool xvec = p.xs_h == 1 && (((uintptr_t)xr) & 15u) == 0;
    constexpr int kXPass = (512 * STEPS + 8 * NT - 1) / (8 * NT);
    constexpr bool kXTail = 8 * NT * kXPass != 512 * STEPS;
    auto quant8 = [&](const uint32_t (&v)[8], int h0) {
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = max(amax, v[i] & 0x7fffu);
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
        const int xs = group_exponent(amax << 16);
        const E2m1Thresholds xth = e2m1_thresholds(xs);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(v[i] << 16, xth) << (4 * i);
        reinterpret_cast<uint32_t*>(xcode)[h0 / 8] = word;
        if ((tid & 3) == 0) xscale[h0 / 32] = (uint8_t)(xs + 127);
    };
    // the row's chunks (8 values) h0 = 8 tid + 8 NT q into registers; with
    // the RMSNorm folded in, also their norm weights
    i32x4_t xv[kXPass];
    float nwv[kXPass][8];
#pragma unroll
    for (int q = 0; q < kXPass; ++q) {
        const int h0 = 8 * tid + 8 * NT * q;
        if (kXTail && h0 >= p.H) continue;
        if (xvec) {
            xv[q] = *reinterpret_cast<const i32x4_t*>(xr + h0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xv[q][i] = (int)((uint32_t)xr[(int64_t)(h0 + 2 * i) * p.xs_h] |
                                 ((uint32_t)xr[(int64_t)(h0 + 2 * i + 1) * p.xs_h] << 16));
        }
        if (p.nw) {
#pragma unroll
            for (int i = 0; i < 8; ++i) nwv[q][i] = norm_weight_at(p.nw, p.nw_f32 != 0, p.nws, h0 + i);
        }
    }
    constexpr int steps = STEPS;
#pragma unroll
    for (int u0 = 0; u0 < steps; u0 += kSmallChunk) {
        i32x4_t wv[kSmallChunk][BPW];
#pragma unroll
        for (int u = 0; u < kSmallChunk; ++u) {
            if (u0 + u < steps) {
                const int k = kbase + 128 * (u0 + u) + 32 * kg;
#pragma unroll
                for (int b = 0; b < BPW; ++b) wv[u][b] = *reinterpret_cast<const i32x4_t*>(wr[b] + k / 2);
            }
        }
        // scale byte 4u + kg of the row's window of 4 steps is this lane's
        // for step u; a window is one aligned 16-byte load (H % 2048 == 0;
        // a byte load per step would cost about as much issue time as a
        // weight load)
        i32x4_t sw[kSmallChunk / 4][BPW];
#pragma unroll
        for (int v = 0; v < kSmallChunk / 4; ++v)
            if (u0 + 4 * v < steps)
#pragma unroll
                for (int b = 0; b < BPW; ++b)
                    sw[v][b] = *reinterpret_cast<const i32x4_t*>(sr[b] + kbase / 32 + 4 * (u0 + 4 * v));
        if (u0 == 0) {
            // keep the row's arithmetic behind the weight loads
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kXPass; ++q) __asm__ volatile("" : "+v"(xv[q]));
            float r = 1.f;
            if (p.nw) {
                // RMSNorm folded in, in the norm kernels' order: the raw row
                // goes to LDS (the reduction buffer, unused until the end),
                // wave 0 sums its squares, and every thread scales its chunks
                uint4* xrow = reinterpret_cast<uint4*>(&red[0][0][0][0]);
#pragma unroll
                for (int q = 0; q < kXPass; ++q) {
                    if (kXTail && 8 * tid + 8 * NT * q >= p.H) continue;
                    xrow[tid + NT * q] = make_uint4((uint32_t)xv[q][0], (uint32_t)xv[q][1], (uint32_t)xv[q][2],
                                                    (uint32_t)xv[q][3]);
                }
                __syncthreads();
                if (w == 0) {
                    const float ss = row_sumsq_chunks(xrow, p.H / 8);
                    if (lane == 0) rsc = rms_scale(ss, p.H, p.eps);
                }
                __syncthreads();
                r = rsc;
            }
#pragma unroll
            for (int q = 0; q < kXPass; ++q) {
                if (kXTail && 8 * tid + 8 * NT * q >= p.H) continue;
                uint32_t v[8];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t u = (uint32_t)xv[q][h];
                    if (p.nw) {
                        v[2 * h] = f32_to_bf16_bits((bf16_lo(u) * r) * nwv[q][2 * h]);
                        v[2 * h + 1] = f32_to_bf16_bits((bf16_hi(u) * r) * nwv[q][2 * h + 1]);
                    } else {
                        v[2 * h] = u & 0xffffu;
                        v[2 * h + 1] = u >> 16;
                    }
                }
                quant8(v, 8 * tid + 8 * NT * q);
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < kSmallChunk; ++u) {
            if (u0 + u < steps) {
                const int k = kbase + 128 * (u0 + u) + 32 * kg;
                const uint4 fa = xcode[k / 32];
                const int asc = xscale[k / 32];
                const i32x8_t a8 = {(int)fa.x, (int)fa.y, (int)fa.z, (int)fa.w, 0, 0, 0, 0};
#pragma unroll
                for (int b = 0; b < BPW; ++b) {
                    const i32x8_t b8 = {wv[u][b][0], wv[u][b][1], wv[u][b][2], wv[u][b][3], 0, 0, 0, 0};
                    const int bsc = (int)((uint32_t)sw[u / 4][b][u % 4] >> (8 * kg));
                    acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[b], 4, 4, 0, bsc, 0, asc);
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        __asm__ volatile("" : "+v"(acc[b]));
#pragma unroll
        for (int i = 0; i < 4; ++i) red[qk][b0 + b][i][lane] = acc[b][i];
    }
    __syncthreads();
    if (w != 0) return;
    // lane (r16, kg) holds h columns 4 kg + i (block 0 / 2) and 16 + 4 kg + i
    // (block 1 / 3); every r16 holds the same values
    float h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float g = 0.f, uu = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                g += red[q][half][i][lane];
                uu += red[q][2 + half][i][lane];
            }
            h[half * 4 + i] = silu_mul(g, uu);
        }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, __float_as_uint(h[i]) & 0x7fffffffu);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
    const int s = group_exponent(amax);
    const E2m1Thresholds th = e2m1_thresholds(s);
    if (r16 != 0) return;
    uint8_t* rp = p.hq + (int64_t)a * (p.I / 2) + c0 / 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        uint32_t v2 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) v2 |= e2m1_code(__float_as_uint(h[half * 4 + i]), th) << (4 * i);
        *reinterpret_cast<uint16_t*>(rp + (16 * half + 4 * kg) / 2) = (uint16_t)v2;
    }
    if (kg == 0) p.hs[(int64_t)a * (p.I / 32) + c0 / 32] = (uint8_t)(s + 127);
}

// bf16 gemm1 for a few tokens, without the align: the bf16 counterpart of
// the kernel above. Workgroup (slot a, h columns c0 .. c0 + 15): 4 waves take
// K = H in quarters, each chaining 16x16x32 MFMAs over its quarter in
// ascending 32-steps from zero (gate rows c0 .. c0 + 15 in block 0, up rows
// in block 1); partial sums added in wave order from zero, SiLU(g) * u
// rounded to bf16 once: the arithmetic of the bf16 weight stream with a
// 4-way K split, so h is bit-identical to it. The token row is staged in LDS;
// a wave streams its weights in chunks of 8 steps (16 KB per wave), the next
// chunk's loads issued before the current chunk's MFMAs.
// NCH: chunks per wave, H / 1024 (even: the row is staged 2048 values per
// pass).
template <int NCH>
__global__ __launch_bounds__(256) void gemm1_small_bf16_kernel(Gemm1SmallParams p) {
    __shared__ i32x4_t xs[kSmallMaxH / 8];           // the token row, 8 bf16 per entry
    __shared__ float red[4][2][4][64];
    __shared__ float rsc;                            // the row's RMSNorm scale
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int ncb = p.I / 16;
    const int a = (int)(blockIdx.x / (uint32_t)ncb);
    const int c0 = (int)(blockIdx.x % (uint32_t)ncb) * 16;
    if (a >= p.A) return;
    const int64_t t = a / p.k, j = a % p.k;
    const int64_t e = (int64_t)p.ids[t * p.is_t + j * p.is_j] - p.e_off;
    if (e < 0 || e >= p.E) return;                   // the same for the whole workgroup
    constexpr int kq = NCH * 256;                    // this wave's quarter of K
    const int kbase = w * kq;
    const uint8_t* wr[2] = {p.gate + e * p.g_e + (int64_t)(c0 + r16) * p.g_r,
                            p.up + e * p.u_e + (int64_t)(c0 + r16) * p.u_r};
    f32x4_t acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float z;
        __asm__("v_mov_b32 %0, 0" : "=v"(z));
        acc[b] = f32x4_t{z, z, z, z};
    }
    // the row: a contiguous one is loaded ahead of the weights, its wait
    // covering only itself
    constexpr int XP = NCH / 2;
    const uint16_t* xr = p.x + t * p.xs_t;
    const bool xvec = p.xs_h == 1 && (((uintptr_t)xr) & 15u) == 0;
    i32x4_t xv[XP];
    if (xvec) {
#pragma unroll
        for (int q = 0; q < XP; ++q) xv[q] = *reinterpret_cast<const i32x4_t*>(xr + 8 * tid + 2048 * q);
    }
    // RMSNorm folded in: the weights of this thread's chunks
    float nwv[XP][8];
    if (p.nw) {
#pragma unroll
        for (int q = 0; q < XP; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i) nwv[q][i] = norm_weight_at(p.nw, p.nw_f32 != 0, p.nws, 8 * tid + 2048 * q + i);
    }
    i32x4_t wv[2][8][2];
    auto load_chunk = [&](int buf, int c) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const int k = kbase + 256 * c + 32 * st + 8 * kg;
#pragma unroll
            for (int b = 0; b < 2; ++b) wv[buf][st][b] = *reinterpret_cast<const i32x4_t*>(wr[b] + 2 * k);
        }
    };
    load_chunk(0, 0);
    if (xvec) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < XP; ++q) __asm__ volatile("" : "+v"(xv[q]));
#pragma unroll
        for (int q = 0; q < XP; ++q) xs[tid + 256 * q] = xv[q];
    } else {
        for (int h0 = 8 * tid; h0 < p.H; h0 += 8 * 256) {
            i32x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (int)((uint32_t)xr[(int64_t)(h0 + 2 * i) * p.xs_h] |
                             ((uint32_t)xr[(int64_t)(h0 + 2 * i + 1) * p.xs_h] << 16));
            xs[h0 / 8] = v;
        }
    }
    __syncthreads();
    if (p.nw) {
        // the row normalised in place, in the norm kernels' order: the sum of
        // squares by wave 0, then each thread its own chunks
        if (w == 0) {
            const float ss = row_sumsq_chunks(reinterpret_cast<const uint4*>(xs), p.H / 8);
            if (lane == 0) rsc = rms_scale(ss, p.H, p.eps);
        }
        __syncthreads();
        const float r = rsc;
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int c = tid + 256 * q;
            const i32x4_t v = xs[c];
            i32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t u = (uint32_t)v[i];
                o[i] = (int)((uint32_t)f32_to_bf16_bits((bf16_lo(u) * r) * nwv[q][2 * i]) |
                             ((uint32_t)f32_to_bf16_bits((bf16_hi(u) * r) * nwv[q][2 * i + 1]) << 16));
            }
            xs[c] = o;
        }
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c + 1 < NCH) load_chunk((c + 1) & 1, c + 1);
        __builtin_amdgcn_sched_barrier(0);           // the next chunk's loads stay ahead
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const int k = kbase + 256 * c + 32 * st + 8 * kg;
            const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, xs[k / 8]);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[c & 1][st][b]), xa,
                                                                 acc[b], 0, 0, 0);
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        __asm__ volatile("" : "+v"(acc[b]));
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][b][i][lane] = acc[b][i];
    }
    __syncthreads();
    if (w != 0) return;
    // lane (r16, kg) holds h columns 4 kg + i; every r16 the same
    uint32_t hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float g = 0.f, uu = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g += red[q][0][i][lane];
            uu += red[q][1][i][lane];
        }
        hb[i] = f32_to_bf16_bits(silu_mul(g, uu));
    }
    if (r16 != 0) return;
    uint16_t* hrow = reinterpret_cast<uint16_t*>(p.hq) + (int64_t)a * p.I + c0 + 4 * kg;
    *reinterpret_cast<uint2*>(hrow) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
}

// bf16 gemm2 and combine in one pass, for a few tokens: one workgroup of 16
// waves per token t and 16 output columns n0 .. n0 + 15. Wave w takes K
// quarter w % 4 of slot j0 + w / 4 for each round of 4 slots j0 = 0, 4, ...:
// 16x16x32 MFMAs chained over the quarter in ascending 32-steps from zero,
// the 4 partial sums added in quarter order from zero and rounded to bf16 -
// the bf16 weight stream's gemm2 with a 4-way K split - then w_tj * y added
// over j in slot order with fmaf as the separate combine does; so the output
// is bit-identical to those two, without y in memory.
// STEPS: 32-steps per K quarter, I / 128.
template <int STEPS>
__global__ __launch_bounds__(1024) void gemm2_combine_bf16_kernel(Gemm2CombineParams q) {
    const GemmParams& p = q.g;
    const CombineParams& c = q.c;
    __shared__ float red[4][4][4][64];
    __shared__ float ys[kG2cMaxK][16];
    __shared__ float wts[kG2cMaxK];
    __shared__ int eid[kG2cMaxK];                    // local expert, or -1
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qk = w & 3, sl = w >> 2;
    const int r16 = lane & 15, kg = lane >> 4;
    const int ncb = p.N / 16;
    const int64_t t = blockIdx.x / (uint32_t)ncb;
    const int n0 = (int)(blockIdx.x % (uint32_t)ncb) * 16;
    if (t >= c.T) return;
    if (threadIdx.x < c.k) {
        const int j = threadIdx.x;
        const int64_t e = (int64_t)c.ids[t * c.is_t + (int64_t)j * c.is_j] - c.e_off;
        eid[j] = e >= 0 && e < c.E ? (int)e : -1;
        wts[j] = c.w[t * c.ws_t + (int64_t)j * c.ws_j];
    }
    __syncthreads();
    const int kbase = qk * STEPS * 32;
    for (int j0 = 0; j0 < c.k; j0 += 4) {
        const int j = j0 + sl;
        const int64_t e = j < c.k ? __builtin_amdgcn_readfirstlane(eid[j]) : -1;
        f32x4_t acc;
        {
            float z;
            __asm__("v_mov_b32 %0, 0" : "=v"(z));
            acc = f32x4_t{z, z, z, z};
        }
        if (e >= 0) {
            const char* wr = reinterpret_cast<const char*>(p.b0) + (e * p.b0_e + (int64_t)(n0 + r16) * p.b0_r) * 2;
            const char* hr = reinterpret_cast<const char*>(p.a) + (t * c.k + j) * p.a_row * 2;
            i32x4_t fb[STEPS], fa[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const int k = kbase + 32 * st + 8 * kg;
                fb[st] = *reinterpret_cast<const i32x4_t*>(wr + 2 * k);
                fa[st] = *reinterpret_cast<const i32x4_t*>(hr + 2 * k);
            }
            __builtin_amdgcn_sched_barrier(0);       // every load issued before the first wait
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[st]),
                                                              __builtin_bit_cast(bf16x8_t, fa[st]), acc, 0, 0, 0);
        }
        __asm__ volatile("" : "+v"(acc));
#pragma unroll
        for (int i = 0; i < 4; ++i) red[qk][sl][i][lane] = acc[i];
        __syncthreads();
        // lane (r16, kg) holds columns 4 kg + i; every r16 the same
        if (qk == 0 && e >= 0 && r16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y = 0.f;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) y += red[qq][sl][i][lane];
                ys[j][4 * kg + i] = bf16_bits_to_f32(f32_to_bf16_bits(y));
            }
        }
        __syncthreads();
    }
    if (w != 0 || lane >= 16) return;
    float out_acc = 0.f;
    for (int j = 0; j < c.k; ++j)
        if (eid[j] >= 0) out_acc = __builtin_fmaf(wts[j], ys[j][lane], out_acc);
    c.out[t * c.os_t + (int64_t)(n0 + lane) * c.os_h] = (uint16_t)f32_to_bf16_bits(out_acc);
}

}  // namespace

hipError_t launch_gemm1_small(const Gemm1SmallParams& p, hipStream_t s) {
    if (p.H % 2048 != 0 || p.H > kSmallMaxH || p.I % 32 != 0) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)p.A * (p.I / 32);
    if (grid == 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256 * (4 / kSmallBPW));
    switch (p.H / 512) {
        case 4: hipLaunchKernelGGL((gemm1_small_kernel<4, kSmallBPW>), g, b, 0, s, p); break;
        case 8: hipLaunchKernelGGL((gemm1_small_kernel<8, kSmallBPW>), g, b, 0, s, p); break;
        case 12: hipLaunchKernelGGL((gemm1_small_kernel<12, kSmallBPW>), g, b, 0, s, p); break;
        default: hipLaunchKernelGGL((gemm1_small_kernel<16, kSmallBPW>), g, b, 0, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm1_small_bf16(const Gemm1SmallParams& p, hipStream_t s) {
    if (p.H % 2048 != 0 || p.H > kSmallMaxH || p.I % 16 != 0) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)p.A * (p.I / 16);
    if (grid == 0) return hipSuccess;
    switch (p.H / 1024) {
        case 2: hipLaunchKernelGGL(gemm1_small_bf16_kernel<2>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
        case 4: hipLaunchKernelGGL(gemm1_small_bf16_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
        case 6: hipLaunchKernelGGL(gemm1_small_bf16_kernel<6>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL(gemm1_small_bf16_kernel<8>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
    }
    return hipGetLastError();
}

bool gemm2_combine_bf16_supported(int64_t I) {
    return I % 128 == 0 && I / 128 >= 4 && I / 128 <= 12 && (I / 128) % 2 == 0;
}

hipError_t launch_gemm2_combine_bf16(const Gemm2CombineParams& p, hipStream_t s) {
    if (!gemm2_combine_bf16_supported(p.g.K) || p.g.N % 16 != 0 || p.c.k > kG2cMaxK) return hipErrorInvalidValue;
    const int64_t grid = p.c.T * (int64_t)(p.g.N / 16);
    if (grid == 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(1024);
    switch (p.g.K / 128) {
        case 4: hipLaunchKernelGGL(gemm2_combine_bf16_kernel<4>, g, b, 0, s, p); break;
        case 6: hipLaunchKernelGGL(gemm2_combine_bf16_kernel<6>, g, b, 0, s, p); break;
        case 8: hipLaunchKernelGGL(gemm2_combine_bf16_kernel<8>, g, b, 0, s, p); break;
        case 10: hipLaunchKernelGGL(gemm2_combine_bf16_kernel<10>, g, b, 0, s, p); break;
        default: hipLaunchKernelGGL(gemm2_combine_bf16_kernel<12>, g, b, 0, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm2_combine(const Gemm2CombineParams& p, hipStream_t s) {
    if (p.g.K != 4 * 128 || p.g.N % 16 != 0 || p.c.k > kG2cMaxK) return hipErrorInvalidValue;
    const int64_t grid = p.c.T * (int64_t)(p.g.N / 16);
    if (grid == 0) return hipSuccess;
    // two slots per wave (one per wave measured no faster at any T), at
    // most 16 waves
    const int W = std::min((p.c.k + 1) / 2, 16);
    const dim3 block(64 * W);
    if (2 * W < p.c.k)
        hipLaunchKernelGGL((gemm2_combine_kernel<2, true>), dim3((unsigned)grid), block, 0, s, p);
    else
        hipLaunchKernelGGL((gemm2_combine_kernel<2, false>), dim3((unsigned)grid), block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmKernelId& id, const GemmParams& p, hipStream_t s) {
    GemmFn fn = lookup(id);
    if (!fn) return hipErrorInvalidValue;
    if (id.nt != 1) {
        // K must be exactly one 4-step ring round; N whole 256-column tiles
        if (p.K != 4 * 128 || p.N % 256 != 0) return hipErrorInvalidValue;
        const int64_t groups = (p.N / 256 + id.nt - 1) / id.nt;
        const int64_t grid = groups * (int64_t)p.max_mblocks;
        if (grid == 0) return hipSuccess;
        hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int tile_n = gemm_tile_n(id);
    const int n_tiles = p.N / tile_n;
    const int G = p.n_tile_groups;
    const int64_t groups = (n_tiles + G - 1) / G;
    const int64_t grid = groups * (int64_t)p.max_mblocks * G;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
