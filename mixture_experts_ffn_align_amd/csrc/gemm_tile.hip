// Grouped expert GEMMs of the fused MoE forward, LDS-tiled variant for many
// tokens per expert.
//
// Same two stages and epilogues as the weight-streaming kernels (stage 1:
// gathered x rows times gate_e^T and up_e^T, then h = SiLU(g) * u; stage 2: h
// rows times w2_e^T scattered to the flat assignment index), but organised
// for reuse instead of streaming: when an expert owns hundreds of rows, every
// weight byte feeds several row blocks, so the chip is bound by the matrix
// cores, the LDS and the L2, not by HBM (ROCm/aiter PR "TP2 MXFP4 fused-MoE
// configs for Qwen3.5-397B", Details: larger block_m for the large token
// buckets).
//
// A workgroup of NW wave64s owns BM rows of one expert times BW weight rows
// (stage 1: BW/2 gate + BW/2 up rows -> BW/2 h columns; stage 2: BW output
// columns); each wave multiplies 64 rows by 128 weight rows (4 x 8 MFMA
// blocks of 16 x 16, accumulators in 128 registers), so one k-step reads 12
// fragments from LDS for 32 MFMAs. K advances in stages of 64 bytes per row
// (32 bf16 or 128 e2m1 values), SUBS = 1 or 2 MFMA k-steps per stage of
// 64 SUBS bytes per row.
//
// Loads go straight from global memory to LDS (global_load_lds_dwordx4, no
// registers, no LDS write instructions): one wave instruction fills 1 KB of
// LDS, 8 tile rows x 128 bytes (SUBS = 2: a whole cache line per 8 lanes) or
// 16 rows x 64 bytes (SUBS = 1: each quad of lanes reads one row's 64
// contiguous bytes). 4 / SUBS stage buffers rotate, the loads of the stage
// 4 / SUBS - 1 ahead are issued while a stage is multiplied, and one
// workgroup barrier per stage publishes a landed stage and retires a consumed
// one. The 8-wave bf16 shapes run the two waves of each SIMD half a stage
// apart instead (two barriers per stage): one multiplies from registers while
// the other reads its fragments, so the matrix core is never left waiting
// for a whole workgroup's LDS reads after a barrier.
//
// Epilogues. The weight fragment is the MFMA's first operand, so a lane's
// accumulator holds 4 consecutive output columns of one row. h and y rows go
// out through a small wave-private LDS patch and leave as 16-byte stores
// that fill whole cache lines; y, read once by the combine much later, is
// stored non-temporally.
//
// LDS layout. Rows are stored row-major, the 16-byte chunk c of tile row r at
// chunk position c ^ g(r): g(r) = (r / 2) ^ (r / 8) (mod 4) for 64-byte rows
// and (r / 2) ^ 4 (r % 2) (mod 8) for 128-byte rows (r mod 16). An MFMA
// fragment (lane l: row l % 16, chunk l / 16 of its k-step) then reads 8
// distinct 16-byte bank groups of a 128-byte bank row in every 8 lanes and
// 16 distinct ones of a 256-byte row in every 16 lanes, so a 16-byte LDS read
// is conflict-free whether the LDS serves 8 or 16 lanes per pass; the loads
// choose which chunk each lane fetches so that the lane order of the LDS
// write is the swizzled order.
//
// Workgroups walk the tiles in expert-major order (see the tile mapping in
// the kernel), cut into one contiguous range per XCD, so the row blocks of an
// expert stream its weight tiles through one XCD's L2 together (the token
// rows, a few MB, are re-read once per weight tile from the L2 / MALL).
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlock = 1024;       // bytes one load instruction writes
constexpr int kScStep = 4;         // e8m0 bytes of one row per k-step

typedef __attribute__((address_space(3))) void* lds_ptr_t;


// BM rows x BW weight rows per workgroup of NW waves, SUBS k-steps of
// 64 bytes per row per stage, NBUF stage buffers; a wave multiplies 16 WMI
// rows by 128 weight rows
template <int MODE, int BM, int BW, int NW, int SUBS, int NBUF>
struct TileShape {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kRowBytes = 64 * SUBS;
    static constexpr int kRowsPerLoad = kBlock / kRowBytes;
    static constexpr int kNBuf = NBUF;
    static_assert(NBUF == 2 || NBUF == 4, "two or four stage buffers");
    static constexpr int kWN = BW / 128;                   // waves along weight rows
    static constexpr int kWM = NW / kWN;                   // waves along rows
    static constexpr int kWMI = BM / (16 * kWM);           // row blocks per wave
    static_assert(kWM * kWN == NW && kWMI * 16 * kWM == BM && kWMI >= 1 && kWMI <= 5, "wave grid");
    static constexpr int kRows = BM + BW;
    static constexpr int kLoads = kRows / (kRowsPerLoad * NW);   // 1 KB loads per wave per stage
    static_assert(kLoads * kRowsPerLoad * NW == kRows, "whole loads");
    // 4-byte scale loads per thread per k-step (MXFP4)
    static constexpr int kScLoads = MODE == 1 ? (kRows + kThreads - 1) / kThreads : 0;
    static constexpr int kScOff = kRows * kRowBytes;
    static constexpr int kScPlane = kScLoads * kThreads * kScStep;   // one k-step's scales
    static constexpr int kBuf = kScOff + SUBS * kScPlane;
};

// 16-byte chunk position of chunk c in tile row r (rows of 64 or 128 bytes;
// see the LDS layout above)
template <int CPR>
__device__ __forceinline__ int swz_t(int r, int c) {
    if (CPR == 4) return (c ^ (r >> 1) ^ (r >> 3)) & 3;
    return (c ^ ((r >> 1) ^ ((r & 1) << 2))) & 7;
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding; expcnt not waited)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

template <int MODE, int STAGE, int BM, int BW, int NW, int SUBS, int NBUF, bool PP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_tile(GemmParams p) {
    using TS = TileShape<MODE, BM, BW, NW, SUBS, NBUF>;
    constexpr int kLoads = TS::kLoads, kScLoads = TS::kScLoads, BUF = TS::kBuf, kWN = TS::kWN;
    constexpr int kRowBytes = TS::kRowBytes, RPL = TS::kRowsPerLoad, WMI = TS::kWMI;
    auto swz = [](int r, int c) { return swz_t<kRowBytes / 16>(r & 15, c); };
    // one array per stage buffer, so the compiler sees that reading one
    // buffer does not depend on the loads still landing in another
    __shared__ __attribute__((aligned(16))) char lds0[BUF];
    __shared__ __attribute__((aligned(16))) char lds1[BUF];
    __shared__ __attribute__((aligned(16))) char lds2[NBUF == 4 ? BUF : 16];
    __shared__ __attribute__((aligned(16))) char lds3[NBUF == 4 ? BUF : 16];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: addresses in SGPRs
    const int wm = w / kWN, wn = w % kWN;
    const int r16 = lane & 15, kg = lane >> 4;

    // ---- tile mapping
    constexpr int tile_cols = STAGE == 1 ? BW / 2 : BW;
    const int n_tiles = p.N / tile_cols;
    // Logical tiles in expert-major order: for each expert, its weight tiles
    // in turn, and for each weight tile the expert's row blocks, so the row
    // blocks that share a weight tile run together and the weight tiles that
    // share those row blocks run next to them. Workgroup b runs on XCD b % 8
    // (the dispatcher deals workgroups to the XCDs in turn) as that XCD's
    // j-th, j = b / 8; the logical tiles are cut into 8 equal contiguous
    // ranges, one per XCD, so an expert's tiles share one L2 and every XCD
    // gets the same number of real tiles. The grid is sized by the sorted
    // capacity; the real block count (the padded length the align wrote) is
    // only known here, so workgroups past the real tiles leave at once.
    const int n_blocks = __builtin_amdgcn_readfirstlane(*p.n_padded) / BM;
    const uint32_t total = (uint32_t)n_blocks * (uint32_t)n_tiles;
    const uint32_t per_xcd = (total + 7u) / 8u;
    const uint32_t xcd = blockIdx.x & 7u, j = blockIdx.x >> 3;
    if (j >= per_xcd) return;
    const uint32_t L = xcd * per_xcd + j;
    if (L >= total) return;
    // expert e owns blocks [b0, b0 + nb) and logical tiles
    // [b0 * n_tiles, (b0 + nb) * n_tiles), so block L / n_tiles is one of its
    const int eo = __builtin_amdgcn_readfirstlane(p.block_expert[L / (uint32_t)n_tiles]);
    const int b0 = __builtin_amdgcn_readfirstlane(p.expert_block[eo]);
    const int nb = __builtin_amdgcn_readfirstlane(p.expert_block[eo + 1]) - b0;
    const uint32_t r = L - (uint32_t)b0 * (uint32_t)n_tiles;
    const int nt = (int)(r / (uint32_t)nb);
    const int mb = b0 + (int)(r % (uint32_t)nb);
    const int e = eo;
    const int row0 = mb * BM;
    const int n0 = nt * tile_cols;
    // Sentinel rows fill only the end of an expert's last block, so the
    // wave's 16-row groups that hold an assignment are a prefix, found from
    // each group's first row; the wave skips the fragment reads and MFMAs of
    // the others (their accumulators stay 0 and the epilogue stores no
    // padding row). A block without padding runs a copy of the pipeline with
    // no such tests.
    int nlive = 0;
#pragma unroll
    for (int mi = 0; mi < TS::kWMI; ++mi)
        nlive += __builtin_amdgcn_readfirstlane(p.sorted[row0 + (wm * TS::kWMI + mi) * 16]) < p.A ? 1 : 0;

    // stage 1 gathers the token row t = a / k, stage 2 the h row of the flat
    // assignment a; a padding row re-reads row 0
    auto a_row_of = [&](int row) -> int64_t {
        const int a = p.sorted[row];
        if (a >= p.A) return 0;
        return STAGE == 1 ? (int64_t)((unsigned)a / (unsigned)p.k) : (int64_t)a;
    };
    constexpr int EB = MODE == 0 ? 2 : 1;   // bytes per stride unit

    // ---- load i of wave w fills LDS block j = w + NW i (tile rows RPL j ..
    // +RPL; [0, BM) are A rows, [BM, BM + BW) weight rows). Lane l writes
    // position l of the block: local row l / (64 / RPL), chunk position
    // p = l % (64 / RPL), so it fetches the chunk that the swizzle stores
    // there. A or weight, gate or up, is the same for the whole wave, so each
    // load has a wave-uniform base and a 32-bit per-lane offset (the host
    // keeps every operand offset below 2^31 bytes).
    constexpr int CPR = kRowBytes / 16;   // 16-byte chunks per row
    const int lr = lane / CPR;
    const int lchunk = swz(RPL * (w % (16 / RPL)) + lr, lane % CPR);
    const char* ld_base[kLoads];
    uint32_t ld_off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int j = w + NW * i;
        const int t = RPL * j + lr;   // tile row
        if (RPL * j < BM) {
            ld_base[i] = reinterpret_cast<const char*>(p.a);
            ld_off[i] = (uint32_t)(a_row_of(row0 + t) * p.a_row * EB);
        } else {
            const int R = t - BM;
            const bool second = STAGE == 1 && RPL * j - BM >= BW / 2;
            const int wrow = n0 + (STAGE == 1 ? R % (BW / 2) : R);
            ld_base[i] =
                reinterpret_cast<const char*>(second ? p.b1 : p.b0) + (int64_t)e * (second ? p.b1_e : p.b0_e) * EB;
            ld_off[i] = (uint32_t)((int64_t)wrow * (second ? p.b1_r : p.b0_r) * EB);
        }
        ld_off[i] += lchunk * 16;
    }
    // MXFP4: 4-byte scale loads, thread t of load j covers tile row
    // t + kThreads j (LDS position = that row; past the last row it re-reads
    // the last row into a slot nobody reads). A wave's 64 rows can straddle
    // the A / weight boundary, so each lane forms its own address.
    const uint8_t* sc_src[kScLoads > 0 ? kScLoads : 1];
    if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < kScLoads; ++j) {
            const int t = min((int)threadIdx.x + TS::kThreads * j, TS::kRows - 1);
            if (t < BM) {
                sc_src[j] = p.a_sc + a_row_of(row0 + t) * p.a_sc_row;
            } else {
                const int R = t - BM;
                const bool second = STAGE == 1 && R >= BW / 2;
                const int wrow = n0 + (STAGE == 1 ? R % (BW / 2) : R);
                sc_src[j] = (second ? p.b1_sc : p.b0_sc) + (int64_t)e * (second ? p.b1sc_e : p.b0sc_e) +
                            (int64_t)wrow * (second ? p.b1sc_r : p.b0sc_r);
            }
        }
    }

    const int S = p.K / (MODE == 0 ? 32 : 128) / SUBS;   // stages; the host keeps it a multiple of kNBuf

    // issue the loads of stage s (clamped: past the end the last stage is
    // loaded again, into a buffer nobody reads) into buffer buf
    auto issue = [&](char* buf, int s) {
        s = s < S ? s : S - 1;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(ld_base[i] + (ld_off[i] + (uint32_t)(s * kRowBytes))),
                (lds_ptr_t)(buf + (w + NW * i) * kBlock), 16, 0, 0);
        if constexpr (MODE == 1) {
#pragma unroll
            for (int u = 0; u < SUBS; ++u)
#pragma unroll
                for (int j = 0; j < kScLoads; ++j)
                    __builtin_amdgcn_global_load_lds(
                        reinterpret_cast<const void*>(sc_src[j] + (s * SUBS + u) * kScStep),
                        (lds_ptr_t)(buf + TS::kScOff + u * TS::kScPlane + (TS::kThreads * j + 64 * w) * kScStep), 4,
                        0, 0);
        }
    };
    constexpr int kPerStage = kLoads + SUBS * kScLoads;   // vector memory instructions per stage

    // ---- MFMA over one stage: wave (wm, wn) multiplies tile rows
    // wm*64 .. +64 by its 8 weight row blocks
    f32x4_t acc[WMI][8];
#pragma unroll
    for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // tile weight row block of the wave's ni-th column block
    auto b_rb = [&](int ni) {
        if (STAGE == 1) return ni < 4 ? wn * 4 + ni : BW / 32 + wn * 4 + (ni - 4);
        return wn * 8 + ni;
    };
    // fragments of one k-step u of a stage buffer: row block rb of the tile
    // is LDS row 16 rb + r16, chunk 4 u + kg
    struct Frags {
        i32x4_t a[WMI], b[8];
        uint32_t as[WMI], bs[8];
    };
    auto read_frags = [&](const char* buf, int u, Frags& f, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        const int rd = r16 * kRowBytes + swz(r16, 4 * u + kg) * 16;
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi)
            if (FULL || mi < nlive)
                f.a[mi] = *reinterpret_cast<const i32x4_t*>(buf + (wm * WMI + mi) * 16 * kRowBytes + rd);
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
            f.b[ni] = *reinterpret_cast<const i32x4_t*>(buf + (BM + b_rb(ni) * 16) * kRowBytes + rd);
        if constexpr (MODE == 1) {
            // a row's four scale bytes of the k-step form one dword: every
            // lane of the row reads that dword (one address, a broadcast;
            // byte reads of it by lanes kg = 0..3 would conflict) and shifts
            // its own byte kg down, the byte the MFMA takes
            const uint32_t* sb = reinterpret_cast<const uint32_t*>(buf + TS::kScOff + u * TS::kScPlane);
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi)
                if (FULL || mi < nlive) f.as[mi] = sb[(wm * WMI + mi) * 16 + r16] >> (8 * kg);
#pragma unroll
            for (int ni = 0; ni < 8; ++ni) f.bs[ni] = sb[BM + b_rb(ni) * 16 + r16] >> (8 * kg);
        }
    };
    // weight fragment first: the accumulator then holds, in lane l, 4
    // consecutive output columns 4 (l / 16) .. +3 of row l % 16, so the
    // epilogues store 8 or 16 contiguous bytes per lane
    auto mfma_frags = [&](const Frags& f, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi) {
            if (!FULL && mi >= nlive) continue;
#pragma unroll
            for (int ni = 0; ni < 8; ++ni) {
                if constexpr (MODE == 0) {
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.b[ni]),
                                                                          __builtin_bit_cast(bf16x8_t, f.a[mi]),
                                                                          acc[mi][ni], 0, 0, 0);
                } else {
                    const i32x8_t a8 = {f.a[mi][0], f.a[mi][1], f.a[mi][2], f.a[mi][3], 0, 0, 0, 0};
                    const i32x8_t b8 = {f.b[ni][0], f.b[ni][1], f.b[ni][2], f.b[ni][3], 0, 0, 0, 0};
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[mi][ni], 4, 4, 0,
                                                                                   (int)f.bs[ni], 0, (int)f.as[mi]);
                }
            }
        }
    };
    // the K loop, with every row group live (FULL) or with the tests
    auto pipeline = [&](auto full_c) {
        auto compute = [&](const char* buf) {
#pragma unroll
            for (int u = 0; u < SUBS; ++u) {
                Frags f;
                read_frags(buf, u, f, full_c);
                mfma_frags(f, full_c);
            }
        };
        // stage s's loads have landed for every wave and every wave is done with
        // stage s - 1: wait for this wave's loads up to stage s (the later
        // stages stay in flight) and its LDS reads, then meet
        auto publish = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_lgkm<(TS::kNBuf - 2) * kPerStage>();
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };

        // ---- pipeline over kNBuf rotating buffers: stage s in buffer s % kNBuf,
        // stage s + kNBuf - 1 loading into the buffer stage s - 1 used
        if constexpr (PP) {
            // Two wave groups, one wave of each per SIMD, half a stage apart:
            // while one group multiplies from registers, the other reads its next
            // stage's fragments from LDS, so each SIMD's matrix core always has a
            // wave with operands ready. Barriers B0, B1, ... separate phases;
            // group 0 reads stage s in [B2s, B2s+1] and multiplies it in
            // [B2s+1, B2s+2], group 1 reads it in [B2s+1, B2s+2] and multiplies in
            // [B2s+2, B2s+3]. The loads of stage s + kNBuf - 1 go out at B2s from
            // both groups into the buffer of stage s - 1, which both groups
            // finished reading before B2s; every wave waits for its loads of
            // stage s + 1 before B2s+2, the first barrier after which stage s + 1
            // is read.
            static_assert(NW == 8, "one wave of each group per SIMD");
            const bool g1 = w >= NW / 2;
            Frags f[SUBS];
            auto bar = [&]() {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            auto read_stage = [&](const char* buf) {
#pragma unroll
                for (int u = 0; u < SUBS; ++u) read_frags(buf, u, f[u], full_c);
            };
            auto mfma_stage = [&]() {
#pragma unroll
                for (int u = 0; u < SUBS; ++u) mfma_frags(f[u], full_c);
            };
            // group 0, stage s: read buffer rd, refill buffer wr (stage s - 1's)
            auto g0 = [&](const char* rd, char* wr, int s) {
                issue(wr, s + NBUF - 1);
                read_stage(rd);
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm<63>();
                bar();
                mfma_stage();
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm<(NBUF - 2) * kPerStage>();
                bar();
            };
            // group 1, stage s: read buffer b, then refill it with stage s + kNBuf
            auto g1s = [&](char* b, int s) {
                bar();
                read_stage(b);
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm<(NBUF - 2) * kPerStage>();
                bar();
                issue(b, s + NBUF);
                mfma_stage();
            };
            issue(lds0, 0);
            if constexpr (NBUF == 4) {
                issue(lds1, 1);
                issue(lds2, 2);
            }
            wait_vm_lgkm<(NBUF - 2) * kPerStage>();
            bar();   // B0
            if (!g1) {
                for (int s = 0; s < S; s += NBUF) {
                    if constexpr (NBUF == 4) {
                        g0(lds0, lds3, s);
                        g0(lds1, lds0, s + 1);
                        g0(lds2, lds1, s + 2);
                        g0(lds3, lds2, s + 3);
                    } else {
                        g0(lds0, lds1, s);
                        g0(lds1, lds0, s + 1);
                    }
                }
            } else {
                issue(NBUF == 4 ? lds3 : lds1, NBUF - 1);
                for (int s = 0; s < S; s += NBUF) {
                    if constexpr (NBUF == 4) {
                        g1s(lds0, s);
                        g1s(lds1, s + 1);
                        g1s(lds2, s + 2);
                        g1s(lds3, s + 3);
                    } else {
                        g1s(lds0, s);
                        g1s(lds1, s + 1);
                    }
                }
            }
        } else if constexpr (NBUF == 4) {
            issue(lds0, 0);
            issue(lds1, 1);
            issue(lds2, 2);
            for (int s = 0; s < S; s += 4) {
                publish();
                issue(lds3, s + 3);
                compute(lds0);
                publish();
                issue(lds0, s + 4);
                compute(lds1);
                publish();
                issue(lds1, s + 5);
                compute(lds2);
                publish();
                issue(lds2, s + 6);
                compute(lds3);
            }
        } else {
            issue(lds0, 0);
            for (int s = 0; s < S; s += 2) {
                publish();
                issue(lds1, s + 1);
                compute(lds0);
                publish();
                issue(lds0, s + 2);
                compute(lds1);
            }
        }
    };
    if (nlive == WMI)
        pipeline(std::integral_constant<bool, true>{});
    else
        pipeline(std::integral_constant<bool, false>{});
    // drain the loads past the end before the workgroup's LDS is released
    wait_vm_lgkm<0>();

    // ---- epilogues: acc[mi][ni][i] is tile row wm*16*WMI + mi*16 + r16,
    // column 4 kg + i of the ni-th 16-column block; a padding row (flat
    // assignment past A) stores nothing
    auto row_assignment = [&](int mi) { return p.sorted[row0 + wm * 16 * WMI + mi * 16 + r16]; };
    // Rows go out through LDS: a wave writes its 16 rows of one mi block into
    // a private, padded LDS patch in the accumulator layout, reads them back
    // row-contiguous and stores 16 bytes per lane, so one store instruction
    // writes whole 128-byte lines of 2 to 8 rows. Every wave is past its last
    // LDS read of the stage buffers before any patch is written.
    auto through_lds = [&](auto write_patch, auto row_bytes_c, auto store_chunk) {
        constexpr int RB = decltype(row_bytes_c)::value;   // bytes of one patch row
        constexpr int RS = RB + 16;                        // padded LDS row stride
        constexpr int LPR = RB / 16;                       // lanes per row
        constexpr int RPI = 64 / LPR;                      // rows per instruction
        static_assert(RPI * LPR == 64 && 16 * RS * (NW / 2 + NW % 2) <= BUF, "patch fits one stage buffer");
        char* tb = (w < (NW + 1) / 2 ? lds0 : lds1) + (w % ((NW + 1) / 2)) * 16 * RS;
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi) {
            const int am = row_assignment(mi);
            write_patch(mi, tb + r16 * RS);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int it = 0; it < 16 / RPI; ++it) {
                const int R = it * RPI + lane / LPR, c = lane % LPR;
                const i32x4_t v = *reinterpret_cast<const i32x4_t*>(tb + R * RS + c * 16);
                const int a = __shfl(am, R);   // lane R holds row R's assignment
                if (a < p.A) store_chunk(a, c, v);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    };
    if constexpr (STAGE == 1 && MODE == 0) {
        // h by flat assignment: 64 bf16 columns per wave row
        char* h = reinterpret_cast<char*>(p.out);
        through_lds(
            [&](int mi, char* prow) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[mi][j][i], acc[mi][4 + j][i]);
                    *reinterpret_cast<uint2*>(prow + (j * 16 + kg * 4) * 2) =
                        uint2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                }
            },
            std::integral_constant<int, 128>{},
            [&](int a, int c, i32x4_t v) {
                *reinterpret_cast<i32x4_t*>(h + ((int64_t)a * p.N + n0 + wn * 64) * 2 + c * 16) = v;
            });
    } else if constexpr (STAGE == 1 && MODE == 1) {
        uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi) {
            const int a = row_assignment(mi);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // the 32 h columns c0 .. c0 + 31 of one scale group: blocks
                // 2q and 2q + 1, 4 columns per lane, over the 4 lanes kg
                const int c0 = n0 + wn * 64 + q * 32;
                uint32_t b[8];
                uint32_t amax = 0;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        b[jj * 4 + i] =
                            __float_as_uint(silu_mul(acc[mi][2 * q + jj][i], acc[mi][4 + 2 * q + jj][i]));
                        amax = max(amax, b[jj * 4 + i] & 0x7fffffffu);
                    }
                amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
                amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
                const int sx = group_exponent(amax);
                const E2m1Thresholds th = e2m1_thresholds(sx);
                if (a >= p.A) continue;
                uint8_t* rp = hq + (int64_t)a * (p.N / 2);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    // even column in the low nibble
                    const uint32_t w16 = e2m1_code(b[jj * 4], th) | (e2m1_code(b[jj * 4 + 1], th) << 4) |
                                         (e2m1_code(b[jj * 4 + 2], th) << 8) | (e2m1_code(b[jj * 4 + 3], th) << 12);
                    *reinterpret_cast<uint16_t*>(rp + (c0 + jj * 16 + kg * 4) / 2) = (uint16_t)w16;
                }
                if (kg == 0) p.out_sc[(int64_t)a * (p.N / 32) + c0 / 32] = (uint8_t)(sx + 127);
            }
        }
    } else {
        // y rows by flat assignment, 128 columns per wave row, bf16 (RNE)
        constexpr int YB = 2;
        char* y = reinterpret_cast<char*>(p.out);
        through_lds(
            [&](int mi, char* prow) {
#pragma unroll
                for (int ni = 0; ni < 8; ++ni) {
                    const uint2 pk = {
                        bf16x2_bits(acc[mi][ni][0], acc[mi][ni][1]),
                        bf16x2_bits(acc[mi][ni][2], acc[mi][ni][3])};
                    *reinterpret_cast<uint2*>(prow + (ni * 16 + kg * 4) * 2) = pk;
                }
            },
            std::integral_constant<int, 128 * YB>{},
            [&](int a, int c, i32x4_t v) {
                // y is read once, by the combine, long after: stream it past the caches
                __builtin_nontemporal_store(
                    v, reinterpret_cast<i32x4_t*>(y + ((int64_t)a * p.out_row + n0 + wn * 128) * YB + c * 16));
            });
    }
}

// Stages of 128 bytes per row (8 rows x 128 bytes per load, two buffers),
// except MXFP4 with 128- or 256-row blocks: 64 bytes (four buffers; the e2m1
// k-step is four times deeper, so a stage is already long)
template <int MODE, int STAGE, int BM, int BW, int NW, int SUBS = (MODE == 0 || BM <= 64 ? 2 : 1),
          int NBUF = 4 / SUBS, bool PP = (NW == 8 && MODE == 0)>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
    using TS = TileShape<MODE, BM, BW, NW, SUBS, NBUF>;
    const int64_t n_tiles = p.N / (STAGE == 1 ? BW / 2 : BW);
    // a multiple of 8 workgroups, each XCD's share covering an eighth of
    // the tiles the capacity allows
    const int64_t grid = ((int64_t)p.max_mblocks * n_tiles + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_tile<MODE, STAGE, BM, BW, NW, SUBS, NBUF, PP>), dim3((unsigned)grid),
                       dim3(TS::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Tile shapes (rows x weight rows, waves): 0 = 256 x 256 x 8, 1 = 128 x 512 x
// 8, 2 = 64 x 512 x 4, 3 = 32 x 512 x 4, 4 = 64 x 256 x 4 (bf16) or 32 x 256
// x 4 (MXFP4), with four 128-byte stage buffers (three stages in flight)
// where K allows it, 5 = 128 x 256 x 8 (about 64 to 160 rows per expert),
// 6 and 7 = the register-resident MXFP4 gemm2 (256 or 128 rows), 8 = MXFP4
// 256 x 256 x 8 with 128-byte gemm1 stages, 9 = MXFP4 128 x 256 x 8 with
// 128-byte stages, 10 = bf16 320 x 256 x 8 (experts of up to 320 rows in
// one block: a weight tile is staged once for them, where 256-row blocks
// stage it twice for an expert of 257 to 320 rows).
int gemm_tile_rows(int mode, int shape) {
    static const int rows[11] = {256, 128, 64, 32, 64, 128, 256, 128, 256, 128, 320};
    return mode == 1 && shape == 4 ? 32 : rows[shape];
}

// Output columns one tile covers (shapes 6 and 7: gemm2 only, 128 columns
// per step of their column walk; as gemm1 they accept no N)
int gemm_tile_cols(int shape, int stage) {
    if (shape == 6 || shape == 7) return stage == 2 ? 128 : (1 << 30);
    const int bw = (shape == 0 || shape == 4 || shape == 5 || shape == 8 || shape == 9 || shape == 10) ? 256 : 512;
    return stage == 1 ? bw / 2 : bw;
}

// K that is a whole number of stage rotations: two 128-byte stages (four for
// bf16 shape 4), four 64-byte or two 128-byte MXFP4 stages (512 values)
int gemm_tile_k_granule(int mode, int shape) {
    if (mode == 1) return 4 * 128;
    return shape == 4 ? 4 * 64 : 2 * 64;
}

// MXFP4 128 x 512 stages do not fit the LDS with their scales; shapes 6 to
// 9 are MXFP4 only, shape 10 bf16 only
bool gemm_tile_supported(int mode, int shape) {
    if (shape >= 6 && shape <= 9) return mode == 1;
    if (shape == 10) return mode == 0;
    return shape >= 0 && shape <= 5 && !(mode == 1 && shape == 1);
}

hipError_t launch_gemm_tile(int mode, int shape, int stage, const GemmParams& p, hipStream_t s) {
    if (!gemm_tile_supported(mode, shape) || p.N % gemm_tile_cols(shape, stage) != 0 ||
        p.K % gemm_tile_k_granule(mode, shape) != 0)
        return hipErrorInvalidValue;
#define MOE_TILE(MD, BM, BW, NW) \
    return stage == 1 ? launch_one<MD, 1, BM, BW, NW>(p, s) : launch_one<MD, 2, BM, BW, NW>(p, s)
#define MOE_TILE4(MD, BM, BW, NW) \
    return stage == 1 ? launch_one<MD, 1, BM, BW, NW, 2, 4>(p, s) : launch_one<MD, 2, BM, BW, NW, 2, 4>(p, s)
#define MOE_TILE_S(MD, BM, BW, NW, SUBS, NBUF)                                      \
    return stage == 1 ? launch_one<MD, 1, BM, BW, NW, SUBS, NBUF>(p, s) \
                      : launch_one<MD, 2, BM, BW, NW, SUBS, NBUF>(p, s)
    if (shape == 6 || shape == 7) {
        if (mode != 1 || stage != 2) return hipErrorInvalidValue;
        return launch_gemm2_rows(shape == 6 ? 256 : 128, p, s);
    }
    if (mode == 1) {
        // 256 x 256: gemm2 (K = I) runs faster with two 128-byte stages;
        // gemm1 keeps four 64-byte ones (shape 0) or takes two 128-byte ones
        // too (shape 8): a load then reads whole 128-byte lines (8 rows x 128
        // bytes), which the L2 serves about twice as fast as the half lines
        // of 64-byte stages, but only one stage is in flight. Which wins
        // depends on the bucket.
        if (shape == 0)
            return stage == 1 ? launch_one<1, 1, 256, 256, 8>(p, s) : launch_one<1, 2, 256, 256, 8, 2, 2>(p, s);
        if (shape == 8)
            return stage == 1 ? launch_one<1, 1, 256, 256, 8, 2, 2>(p, s) : launch_one<1, 2, 256, 256, 8, 2, 2>(p, s);
        // 128 x 256 with two 128-byte stages (shape 9; shape 5 has four
        // 64-byte ones)
        if (shape == 9) MOE_TILE_S(1, 128, 256, 8, 2, 2);
        if (shape == 2) MOE_TILE(1, 64, 512, 4);
        if (shape == 3) MOE_TILE(1, 32, 512, 4);
        if (shape == 5) MOE_TILE(1, 128, 256, 8);
        // four buffers need four 256-value stages per rotation
        if (p.K % (4 * 256) == 0) MOE_TILE4(1, 32, 256, 4);
        MOE_TILE(1, 32, 256, 4);
    }
    if (shape == 0) MOE_TILE(0, 256, 256, 8);
    if (shape == 1) MOE_TILE(0, 128, 512, 8);
    if (shape == 2) MOE_TILE(0, 64, 512, 4);
    if (shape == 3) MOE_TILE(0, 32, 512, 4);
    if (shape == 5) MOE_TILE(0, 128, 256, 8);
    // 320 rows: the two-group schedule holds two k-steps of fragments on top
    // of the 160 accumulator registers, more than a wave's 256 at two waves
    // per SIMD, so this shape runs the one-barrier pipeline
    if (shape == 10)
        return stage == 1 ? launch_one<0, 1, 320, 256, 8, 2, 2, false>(p, s)
                          : launch_one<0, 2, 320, 256, 8, 2, 2, false>(p, s);
    MOE_TILE4(0, 64, 256, 4);
#undef MOE_TILE
#undef MOE_TILE4
#undef MOE_TILE_S
}

}  // namespace moe
