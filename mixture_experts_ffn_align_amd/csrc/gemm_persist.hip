// MXFP4 gemm1 + SiLU(gate) * up as a persistent weight stream.
//
// What it computes is stage 1 of gemm_stream.hip in MXFP4 mode with the K
// of a row block unsplit: for a sorted block of BM rows of expert e, the
// token rows times gate_e^T and up_e^T, h = SiLU(g) * u quantised per 32
// columns (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for Qwen3.5-397B",
// Details: ActivationType.Silu), stored by flat assignment index. Operands,
// fragment layouts and the order of the MFMAs are the same, so h is the same
// bit for bit.
//
// How it runs differs. A work item is one row block times one tile of
// 32 * NW h columns (wave w: 32 gate + 32 up weight rows); the grid holds one
// workgroup per compute unit, and each workgroup walks a static list of
// items (item_walk below: an XCD's workgroups share one contiguous range of
// them, so the column tiles of a row block and the blocks of an expert run
// side by side on one XCD and share its L2). On this chip a compute unit
// serves one streaming workgroup at a time: a second resident workgroup's
// first loads return only as the first one finishes, so with one workgroup per item every item paid the latency of its
// first loads and the drain of its ring in series. Here each wave's ring of
// U = 4 weight steps runs on from one item into the next: the last round of
// an item refills its slots with the next item's first steps, and everything
// else the next item needs is fetched one item (or one round) ahead:
//  * the experts of all of the workgroup's items, into an LDS table before
//    the first item (inside the loop a load of them would be a vector load,
//    since the h stores may alias it, and its wait would drain the ring);
//  * the next item's sorted entries, in an item's first round; they become
//    row pointers only in its last round, so that no wait before then (the
//    load counter is in order) covers the weight loads in flight;
//  * the next item's weight scale runs (K/32 bytes per weight row), in the
//    first half of an item, two 1 KB loads per round that each read whole
//    runs (R lanes of 16 bytes per row: a load that took 16 bytes of each of
//    64 rows asked for four times the cache lines per byte and cost a tenth
//    of the kernel's time), written to this wave's part of a double-buffered
//    LDS area (each wave reads only its own rows' runs, so no barrier guards
//    them);
//  * the token-row fragments of the next round (one round = 4 steps of 128
//    k), staged in LDS by the four or eight waves together, double-buffered
//    with one barrier per round.
// After the last item the ring re-reads the last step of the current one, so
// every wave issues the same loads each round and the compiler's wait counts
// stay exact.

#include "gemm_persist.h"

namespace moe {
namespace {

// bytes of weight scales per row the LDS runs hold (K / 32 at most): K up
// to 8192 with four waves and blocks of 16 or 32 rows, else 4096 (the
// token-row buffers of 64-row blocks, or the runs of eight waves, take the
// rest of the 160 KB)
template <int NW, int BM>
constexpr int persist_scb() {
    return NW == 4 && BM <= 32 ? 256 : 128;
}
constexpr int kPersistItems = 256;   // items per workgroup at most (the host checks)

// The items of this workgroup: first, first + step, ... below end. Workgroup
// g runs on XCD g % 8 (the dispatcher deals workgroups to the 8 XCDs in
// turn) as that XCD's (g / 8)-th; the items are cut into 8 contiguous
// ranges, one per XCD, and an XCD's workgroups deal its range among
// themselves, so items next to each other in order (the column tiles of one
// row block: the same token rows; the row blocks of one expert: the same
// weights) run at the same time on one XCD and meet in its L2 instead of
// crossing to the MALL or HBM once per XCD (gemm1 of the TP2 shard: 1% faster
// than the plain walk g, g + G, ... at 1024 tokens, 2% at 2048). No
// workgroup gets more than ceil(n_items / G) items either way. A grid that
// is not a whole number of workgroups per XCD takes the plain walk.
struct ItemWalk {
    int first, step, end;
};
__device__ __forceinline__ ItemWalk item_walk(int n_items) {
    const int G = (int)gridDim.x, g = (int)blockIdx.x;
    if (G % 8 != 0) return ItemWalk{g, G, n_items};
    const int per = (n_items + 7) / 8;
    const int lo = (g % 8) * per;
    return ItemWalk{lo + g / 8, G / 8, min(n_items, lo + per)};
}

// One work item as a lane sees it.
template <int MB>
struct PItem {
    const char* b[4];        // this lane's weight row in column blocks 0, 1 (gate) and 2, 3 (up)
    const uint8_t* scg;      // the expert's gate and up scales
    const uint8_t* scu;
    const char* a[MB];       // token row r16 of each 16-row group (padding: row 0)
    const uint8_t* as[MB];   // its scale row
    int row[MB];             // flat assignment index of that row (>= A: padding)
    int e;                   // expert
    int n0;                  // the wave's first h column
    int s0;                  // first step (the dummy after the last item re-reads the last round)
};

// Keeps a value of the accumulator chain where it is: in AGPRs with four
// waves (one per SIMD: room for both register files), in VGPRs with eight.
template <int NW>
__device__ __forceinline__ void pin_acc(f32x4_t& v) {
    if constexpr (NW == 4)
        __asm__ volatile("" : "+a"(v));
    else
        __asm__ volatile("" : "+v"(v));
}

template <int BM, int NW, int R>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm1_persist(GemmParams p) {
    constexpr int MB = BM / 16, NB = 4, U = 4;
    constexpr int STEPS = 4 * R;                // 128 k per step, R ring rounds per item
    constexpr int FR = 4 * MB;                  // 1 KB token-row fragments per round: (mi, u)
    constexpr int AR = (FR + NW - 1) / NW;      // fragments one wave stages per round
    constexpr int SCB = persist_scb<NW, BM>();
    static_assert(R % 2 == 0 && STEPS * 4 <= SCB, "scale runs must fit their LDS rows");
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * FR * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[2 * NW * 64 * SCB];
    __shared__ int e_tab[kPersistItems];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int n_tiles = p.N / (32 * NW);
    const int n_items = (*p.n_padded / BM) * n_tiles;
    const ItemWalk wk = item_walk(n_items);
    int it = wk.first;
    if (it >= wk.end) return;

    // an item's first h column and its expert's scales (wave-uniform)
    auto set_item = [&](PItem<MB>& I, int item, int e) {
        I.e = e;
        I.n0 = (item % n_tiles) * (32 * NW) + w * 32;
        I.scg = p.b0_sc + (int64_t)e * p.b0sc_e;
        I.scu = p.b1_sc + (int64_t)e * p.b1sc_e;
    };
    // this lane's weight rows (needed from the item's first refill on)
    auto set_weights = [&](PItem<MB>& I) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const bool up = nb >= 2;
            const int wrow = I.n0 + (nb & 1) * 16 + r16;
            I.b[nb] = reinterpret_cast<const char*>(up ? p.b1 : p.b0) + (int64_t)I.e * (up ? p.b1_e : p.b0_e) +
                      (int64_t)wrow * (up ? p.b1_r : p.b0_r);
        }
    };
    // staging load i of an item's scale runs: rows i * 64 / R .. of the wave
    // (row nb * 16 + rr: column block nb, row rr), R lanes of 16 bytes per row
    constexpr int RPI = 64 / R;
    auto run_row = [&](int i) { return i * RPI + lane / R; };
    auto run_src = [&](const PItem<MB>& I, int i) {
        const int row = run_row(i), nb = row >> 4;
        const bool up = nb >= 2;
        const int wrow = I.n0 + (nb & 1) * 16 + (row & 15);
        return (up ? I.scu : I.scg) + (int64_t)wrow * (up ? p.b1sc_r : p.b0sc_r) + (lane % R) * 16;
    };
    auto run_dst = [&](uint8_t* run, int i) { return run + run_row(i) * SCB + (lane % R) * 16; };
    // the block's sorted entries (loads)
    auto load_rows = [&](PItem<MB>& I, int item) {
        const int mb = item / n_tiles;
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) I.row[mi] = p.sorted[mb * BM + mi * 16 + r16];
    };
    // token-row pointers from the sorted entries (a padding row re-reads row 0)
    auto set_rows = [&](PItem<MB>& I) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const int a = I.row[mi];
            const int64_t t = a < p.A ? (int64_t)((unsigned)a / (unsigned)p.k) : 0;
            I.a[mi] = reinterpret_cast<const char*>(p.a) + t * p.a_row;
            I.as[mi] = p.a_sc + t * p.a_sc_row;
        }
    };
    // this wave's scale runs in buffer b: row r (the order of PItem::sc) at r * SCB
    auto sc_buf = [&](int b) { return sc_lds + (size_t)((b * NW + w) * 64) * SCB; };

    // the experts of this workgroup's items
    const int n_mine = (wk.end - it + wk.step - 1) / wk.step;
    for (int q = threadIdx.x; q < n_mine && q < kPersistItems; q += 64 * NW)
        e_tab[q] = p.block_expert[(it + q * wk.step) / n_tiles];
    __syncthreads();

    PItem<MB> cur;
    set_item(cur, it, e_tab[0]);
    set_weights(cur);
    load_rows(cur, it);
    set_rows(cur);
    cur.s0 = 0;
    int it_n = it + wk.step;

    // ---- the first item's scale runs, whole
    {
        i32x4_t v[R];
#pragma unroll
        for (int i = 0; i < R; ++i) v[i] = *reinterpret_cast<const i32x4_t*>(run_src(cur, i));
#pragma unroll
        for (int i = 0; i < R; ++i) *reinterpret_cast<i32x4_t*>(run_dst(sc_buf(0), i)) = v[i];
    }

    // ---- operand loads
    i32x4_t fb[U][NB];
    auto load_B = [&](int u, const char* const (&b)[NB], int st) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            fb[u][nb] = *reinterpret_cast<const i32x4_t*>(b[nb] + (int64_t)st * 64 + kg * 16);
    };
    i32x4_t areg[AR];
    // fragments f = w, w + NW, ... of the round starting at step st0 (past FR:
    // the last one again, written twice with the same bytes)
    auto load_A = [&](const char* const (&a)[MB], int st0) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            int f = w + NW * i;
            f = f < FR ? f : FR - 1;
            const char* src;
            if constexpr (NW == 4) {
                src = a[i];                    // f = w + 4i: row group i, step w
            } else {
                const int mi = f >> 2;
                src = a[0];
#pragma unroll
                for (int m = 1; m < MB; ++m) src = m == mi ? a[m] : src;
            }
            areg[i] = *reinterpret_cast<const i32x4_t*>(src + (int64_t)(st0 + (f & 3)) * 64 + kg * 16);
        }
    };
    auto store_A = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            int f = w + NW * i;
            f = f < FR ? f : FR - 1;
            *reinterpret_cast<i32x4_t*>(a_lds + (size_t)((buf * FR + f) << 10) + lane * 16) = areg[i];
        }
    };
    // scale windows of the round starting at step st0: 16 bytes per row, byte
    // 4u + kg the scale of step st0 + u for this lane's k group
    uint32_t bsc[NB], asc[MB], bsc_n[NB][U], asc_n[MB][U];
    auto load_windows = [&](const uint8_t* run, const uint8_t* const (&as)[MB], int st0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const i32x4_t v = *reinterpret_cast<const i32x4_t*>(run + (nb * 16 + r16) * SCB + st0 * 4);
#pragma unroll
            for (int u = 0; u < U; ++u) bsc_n[nb][u] = (uint32_t)v[u];
        }
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const i32x4_t v = *reinterpret_cast<const i32x4_t*>(as[mi] + st0 * 4);
#pragma unroll
            for (int u = 0; u < U; ++u) asc_n[mi][u] = (uint32_t)v[u];
        }
    };
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
    f32x4_t acc[MB][NB];
    auto zero_acc = [&]() {
        // zeroed through registers the compiler cannot see as constants, so
        // that every MFMA accumulates in place
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float z;
                __asm__("v_mov_b32 %0, 0" : "=v"(z));
                acc[mi][nb] = f32x4_t{z, z, z, z};
            }
    };
    auto compute = [&](int u, const uint8_t* abuf) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const i32x4_t af = *reinterpret_cast<const i32x4_t*>(abuf + (size_t)((mi * 4 + u) << 10) + lane * 16);
            const i32x8_t a8 = {af[0], af[1], af[2], af[3], 0, 0, 0, 0};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const i32x4_t bv = fb[u][nb];
                const i32x8_t b8 = {bv[0], bv[1], bv[2], bv[3], 0, 0, 0, 0};
                acc[mi][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a8, b8, acc[mi][nb], 4, 4, 0, (int)(asc[mi] >> (8 * u)), 0, (int)(bsc[nb] >> (8 * u)));
            }
        }
        // pinned here (in AGPRs, where the MFMAs accumulate): the rounds are
        // straight-line code, and the compiler would otherwise sink every
        // MFMA to the epilogue and keep all their operands alive until then
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) pin_acc<NW>(acc[mi][nb]);
    };
    // LDS-only workgroup barrier: waits for this wave's LDS accesses, not for
    // the weight loads in flight
    auto lds_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: the first item's ring, first round of token rows, scale windows
#pragma unroll
    for (int u = 0; u < U; ++u) load_B(u, cur.b, u);
    load_A(cur.a, 0);
    store_A(0);
    load_windows(sc_buf(0), cur.as, 0);
    pack_scales();
    zero_acc();

    uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
    int j = 0;
    for (;;) {
        // The next item (after the last one: this one again from its last
        // round, a dummy whose loads are harmless re-reads). Its sorted
        // entries are loaded in round 0 and turned into row pointers only in
        // the last round, so that no wait before then covers the ring.
        const bool has_n = it_n < wk.end;
        const int it_x = has_n ? it_n : it;
        PItem<MB> nxt;
        set_item(nxt, it_x, e_tab[has_n ? j + 1 : j]);
        nxt.s0 = has_n ? 0 : STEPS - 4;
        const uint8_t* run_cur = sc_buf(j & 1);
        uint8_t* run_nxt = sc_buf((j + 1) & 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            lds_barrier();                       // round r's fragments visible; the other buffer idle
            if (r == 0) load_rows(nxt, it_x);
            const uint8_t* abuf = a_lds + (size_t)(((r & 1) * FR) << 10);
            const bool last = r + 1 == R;
            const int st0 = last ? nxt.s0 : 4 * (r + 1);
            if (last) {
                set_rows(nxt);
                set_weights(nxt);
                load_A(nxt.a, st0);
            } else {
                load_A(cur.a, st0);
            }
            // staging loads 2r and 2r + 1 of the next item's scale runs
            i32x4_t sv[2];
            if (r < R / 2) {
#pragma unroll
                for (int t = 0; t < 2; ++t) sv[t] = *reinterpret_cast<const i32x4_t*>(run_src(nxt, 2 * r + t));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                compute(u, abuf);
                __builtin_amdgcn_sched_barrier(0);
                if (last) {
                    load_B(u, nxt.b, st0 + u);
                    if (u == 0) load_windows(run_nxt, nxt.as, st0);
                } else {
                    load_B(u, cur.b, st0 + u);
                    if (u == 0) load_windows(run_cur, cur.as, st0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            pack_scales();
            store_A((r + 1) & 1);
            if (r < R / 2) {
#pragma unroll
                for (int t = 0; t < 2; ++t) *reinterpret_cast<i32x4_t*>(run_dst(run_nxt, 2 * r + t)) = sv[t];
            }
        }

        // ---- epilogue: h = SiLU(g) * u, quantised per 32 columns in
        // registers (max over the 16 lanes of a row), by flat assignment.
        // The MFMAs read operands from every lane: pin their results before
        // the per-row branches below.
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) pin_acc<NW>(acc[mi][nb]);
        const int n0 = cur.n0;
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const f32x4_t g0 = acc[mi][0], g1 = acc[mi][1], u0 = acc[mi][2], u1 = acc[mi][3];
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
                const int a = __shfl(cur.row[mi], kg * 4 + i);   // row kg*4+i of the group
                if (a >= p.A) continue;
                uint8_t* rp = hq + (int64_t)a * (p.N / 2);
                if ((r16 & 1) == 0) {
                    rp[(n0 + r16) / 2] = (uint8_t)(c0 | (o0 << 4));
                    rp[(n0 + 16 + r16) / 2] = (uint8_t)(c1 | (o1 << 4));
                }
                if (r16 == 0) p.out_sc[(int64_t)a * (p.N / 32) + n0 / 32] = (uint8_t)(s + 127);
            }
        }
        zero_acc();
        if (!has_n) break;
        cur = nxt;
        it = it_n;
        it_n = it + wk.step;
        ++j;
    }
}

// MXFP4 gemm2 with K = 512 (I of the TP2 shard: one ring round per tile) as
// a persistent stream. An item is one row block times one 256-column tile
// of w2 (wave w: 64 weight rows); workgroup g takes items g, g + G, ...
// (here the XCD-range walk of gemm1 measured 2-3% slower: its items share
// only a block's few h rows, while the token rows gemm1's neighbours share
// are 2 KB each). Per
// item: the four steps of the ring multiply the item's h fragments (from LDS)
// while their slots are refilled with the next item's four steps; the next
// item's h fragments, h scales and weight scales are loaded at the item's
// start, its sorted entries one item earlier still. Each weight fragment is
// the MFMA's first operand, so a lane holds 4 consecutive output columns of
// one row and stores them as one 8-byte write, exactly as the multi-tile
// stream does (the same MFMA chain: bit-identical y).
template <int BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm2_persist(GemmParams p) {
    constexpr int MB = BM / 16, NB = 4, U = 4;
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * MB * U * 1024];   // buffer, fragment (mi, u)
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[2 * 4 * 1024];       // buffer, wave: 64 rows x 16 B
    // y rows of a wave (64 columns: 128 bytes) on their way out, padded
    constexpr int YP = 144;
    __shared__ __attribute__((aligned(16))) uint8_t y_lds[4 * MB * 16 * YP];
    __shared__ int e_tab[kPersistItems];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int n_tiles = p.N / 256;
    const int n_items = (*p.n_padded / BM) * n_tiles;
    const int G = (int)gridDim.x;
    int it = (int)blockIdx.x;
    if (it >= n_items) return;
    const int n_mine = (n_items - it + G - 1) / G;
    for (int q = threadIdx.x; q < n_mine && q < kPersistItems; q += 256)
        e_tab[q] = p.block_expert[(it + q * G) / n_tiles];
    __syncthreads();

    auto col0 = [&](int item) { return (item % n_tiles) * 256 + w * 64; };   // the wave's first column
    auto load_rows = [&](int (&rows)[MB], int item) {
        const int mb = item / n_tiles;
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) rows[mi] = p.sorted[mb * BM + mi * 16 + r16];
    };
    // h fragment (mi, u = w) of row group mi: wave w stages step w of every group
    i32x4_t areg[MB];
    uint32_t asw[MB][U];      // h scale windows: word u = the 4 k groups' scales of step u
    auto load_A = [&](const int (&rows)[MB]) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const int64_t r = rows[mi] < p.A ? rows[mi] : 0;
            areg[mi] = *reinterpret_cast<const i32x4_t*>(reinterpret_cast<const char*>(p.a) + r * p.a_row +
                                                        w * 64 + kg * 16);
            const i32x4_t v = *reinterpret_cast<const i32x4_t*>(p.a_sc + r * p.a_sc_row);
#pragma unroll
            for (int u = 0; u < U; ++u) asw[mi][u] = (uint32_t)v[u];
        }
    };
    auto store_A = [&](int buf) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
            *reinterpret_cast<i32x4_t*>(a_lds + (size_t)((buf * MB * U + mi * U + w) << 10) + lane * 16) =
                areg[mi];
    };
    // weight scales: row col0 + lane of the tile, one 16-byte run (K / 32)
    i32x4_t bsw;
    auto load_bs = [&](int e, int item) {
        bsw = *reinterpret_cast<const i32x4_t*>(p.b0_sc + (int64_t)e * p.b0sc_e +
                                                (int64_t)(col0(item) + lane) * p.b0sc_r);
    };
    auto store_bs = [&](int buf) {
        *reinterpret_cast<i32x4_t*>(sc_lds + (size_t)((buf * 4 + w) << 10) + lane * 16) = bsw;
    };
    uint32_t asc[MB], bsc[NB];
    auto pack = [&](int buf) {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            uint32_t v = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) v |= ((asw[mi][u] >> (8 * kg)) & 0xffu) << (8 * u);
            asc[mi] = v;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const i32x4_t v =
                *reinterpret_cast<const i32x4_t*>(sc_lds + (size_t)((buf * 4 + w) << 10) + (nb * 16 + r16) * 16);
            uint32_t pk = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) pk |= (((uint32_t)v[u] >> (8 * kg)) & 0xffu) << (8 * u);
            bsc[nb] = pk;
        }
    };
    i32x4_t fb[U][NB];
    auto load_B = [&](int u, int e, int item) {
        const char* base = reinterpret_cast<const char*>(p.b0) + (int64_t)e * p.b0_e;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            fb[u][nb] = *reinterpret_cast<const i32x4_t*>(base + (int64_t)(col0(item) + nb * 16 + r16) * p.b0_r +
                                                          u * 64 + kg * 16);
    };
    f32x4_t acc[MB][NB];
    auto zero_acc = [&]() {
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float z;
                __asm__("v_mov_b32 %0, 0" : "=v"(z));
                acc[mi][nb] = f32x4_t{z, z, z, z};
            }
    };
    auto lds_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: item 0's operands, the next item's sorted entries
    // (the next item's sorted entries go out before the ring: on this path
    // into the loop, as on the loop's own, the weight loads are the newest,
    // so the loop's wait for the entries leaves the ring in flight)
    int rows_c[MB], rows_n[MB];
    load_rows(rows_c, it);
    load_rows(rows_n, n_mine > 1 ? it + G : it);
    int e_c = e_tab[0];
#pragma unroll
    for (int u = 0; u < U; ++u) load_B(u, e_c, it);
    load_A(rows_c);
    load_bs(e_c, it);
    store_A(0);
    store_bs(0);
    lds_barrier();
    pack(0);
    zero_acc();

    uint16_t* y = reinterpret_cast<uint16_t*>(p.out);
    for (int j = 0;; ++j) {
        // the next item (after the last one: this one again, harmless re-reads)
        const bool has_n = j + 1 < n_mine;
        const int it_n = has_n ? it + G : it;
        const int e_n = e_tab[has_n ? j + 1 : j];
        int rows_nn[MB];
        load_A(rows_n);
        load_bs(e_n, it_n);
        load_rows(rows_nn, j + 2 < n_mine ? it + 2 * G : it_n);
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* abuf = a_lds + (size_t)(((j & 1) * MB * U) << 10);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) {
                const i32x4_t af = *reinterpret_cast<const i32x4_t*>(abuf + (size_t)((mi * U + u) << 10) + lane * 16);
                const i32x8_t a8 = {af[0], af[1], af[2], af[3], 0, 0, 0, 0};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const i32x8_t b8 = {fb[u][nb][0], fb[u][nb][1], fb[u][nb][2], fb[u][nb][3], 0, 0, 0, 0};
                    acc[mi][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        b8, a8, acc[mi][nb], 4, 4, 0, (int)(bsc[nb] >> (8 * u)), 0, (int)(asc[mi] >> (8 * u)));
                }
            }
            // pinned before the refill of the slot they read (see the
            // persistent gemm1)
#pragma unroll
            for (int mi = 0; mi < MB; ++mi)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) __asm__ volatile("" : "+a"(acc[mi][nb]));
            __builtin_amdgcn_sched_barrier(0);
            load_B(u, e_n, it_n);
            __builtin_amdgcn_sched_barrier(0);
        }
        // y rows by flat assignment (bf16, RNE). A lane holds columns 4 kg ..
        // +3 of column block nb for row r16; through the wave's LDS patch the
        // 16 rows leave as whole 128-byte lines, 8 lanes of 16 bytes per row
        // (about 5% faster than storing each column block's 32-byte pieces).
        const int c0 = col0(it);
        uint8_t* yp = y_lds + w * (MB * 16 * YP);
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                const u32x2_t pk = {bf16x2_bits(acc[mi][nb][0], acc[mi][nb][1]),
                                    bf16x2_bits(acc[mi][nb][2], acc[mi][nb][3])};
                *reinterpret_cast<u32x2_t*>(yp + (mi * 16 + r16) * YP + nb * 32 + kg * 8) = pk;
            }
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = h * 8 + (lane >> 3), ch = lane & 7;
                const i32x4_t v = *reinterpret_cast<const i32x4_t*>(yp + (mi * 16 + row) * YP + ch * 16);
                const int a = __shfl(rows_c[mi], row);
                if (a < p.A)
                    __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(y + (int64_t)a * p.out_row + c0 + ch * 8));
            }
        zero_acc();
        if (!has_n) break;
        // the next item's h fragments and weight scales to the other buffers
        store_A((j + 1) & 1);
        store_bs((j + 1) & 1);
        lds_barrier();
        pack((j + 1) & 1);
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            rows_c[mi] = rows_n[mi];
            rows_n[mi] = rows_nn[mi];
        }
        it = it_n;
    }
}

template <int BM>
hipError_t launch_g2(const GemmParams& p, hipStream_t s) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t n_items = (int64_t)p.max_mblocks * (p.N / 256);
    const int64_t grid = n_items < cus ? n_items : cus;
    if (grid <= 0) return hipSuccess;
    if (n_items > grid * kPersistItems) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm2_persist<BM>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int BM, int NW, int R>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    // one workgroup per compute unit, never more than there are item slots
    const int64_t n_items = (int64_t)p.max_mblocks * (p.N / (32 * NW));
    const int64_t grid = n_items < cus ? n_items : cus;
    if (grid <= 0) return hipSuccess;
    if (n_items > grid * kPersistItems) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm1_persist<BM, NW, R>), dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool gemm1_persist_supported(int bm, int nw, int64_t K, int64_t N) {
    if (!(bm == 16 || bm == 32 || (bm == 64 && nw == 4)) || !(nw == 4 || nw == 8)) return false;
    const bool k_ok = K == 2048 || K == 4096 || (nw == 4 && bm <= 32 && K == 8192);
    return k_ok && N % (32 * nw) == 0;
}

template <int BM, int NW>
hipError_t launch_r(const GemmParams& p, hipStream_t s) {
    if (p.K == 2048) return launch_one<BM, NW, 4>(p, s);
    if constexpr (NW == 4 && BM <= 32) {
        if (p.K == 8192) return launch_one<BM, NW, 16>(p, s);
    }
    return launch_one<BM, NW, 8>(p, s);
}

bool gemm2_persist_supported(int bm, int64_t K, int64_t N) {
    return (bm == 16 || bm == 32 || bm == 64) && K == 512 && N % 256 == 0;
}

hipError_t launch_gemm2_persist(int bm, const GemmParams& p, hipStream_t s) {
    if (!gemm2_persist_supported(bm, p.K, p.N)) return hipErrorInvalidValue;
    return bm == 16 ? launch_g2<16>(p, s) : (bm == 32 ? launch_g2<32>(p, s) : launch_g2<64>(p, s));
}

hipError_t launch_gemm1_persist(int bm, int nw, const GemmParams& p, hipStream_t s) {
    if (!gemm1_persist_supported(bm, nw, p.K, p.N)) return hipErrorInvalidValue;
    if (bm == 16) return nw == 4 ? launch_r<16, 4>(p, s) : launch_r<16, 8>(p, s);
    if (bm == 64) return launch_r<64, 4>(p, s);
    return nw == 4 ? launch_r<32, 4>(p, s) : launch_r<32, 8>(p, s);
}

}  // namespace moe
