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
// A workgroup is eight wave64s (two per SIMD; four waves, one per SIMD, in
// MXFP4 mode) and owns BM rows of one expert
// times BW weight rows (stage 1: BW/2 gate + BW/2 up rows -> BW/2 h columns;
// stage 2: BW output columns); each wave multiplies 64 rows by 128 weight
// rows (4 x 8 MFMA blocks of 16 x 16, accumulators in 128 VGPRs), so one
// k-step reads 12 fragments from LDS for 32 MFMAs. K advances in stages of
// 128 bytes per row (64 bf16 or 256 e2m1 values), i.e. two MFMA k-steps; the
// LDS holds two stages.
//
// Loads. One wave instruction reads 8 rows x 128 contiguous bytes (lanes
// 8q .. 8q+7 read row q), a whole cache line per 8 lanes: on gfx950 this
// streams from L2 at about three times the rate of the 16 rows x 64 bytes
// that an MFMA fragment spans. The stage goes global -> registers -> LDS, one
// stage ahead of the one being multiplied.
//
// LDS layout. Row-major, 128 bytes per tile row per stage, the 16-byte
// chunk c of row r stored at chunk position c ^ f(r), f(r) = (r/2) ^ 4 (r%2)
// (mod 8). An MFMA fragment (lane l: row l % 16, chunk 4 s + l / 16 for
// k-step s of the stage) and a load instruction (8 rows x 8 chunks) then
// both touch 8 distinct 16-byte bank groups in every 8 lanes and 16 in every
// 16, so neither the writes nor the fragment reads conflict.
//
// Consecutive workgroups are kept on one XCD and cover groups of row blocks x
// weight tiles, so the row blocks of an expert share its weight tiles through
// that XCD's L2 and the weight tiles share the rows.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowBytes = 128;     // bytes of one row per stage
constexpr int kScRow = 8;          // e8m0 bytes of one row per stage

constexpr int WMI = 4;             // row blocks of 16 per wave

// BM rows x BW weight rows per workgroup of NW waves; each wave multiplies
// 64 rows by 128 weight rows
template <int MODE, int BM, int BW, int NW>
struct TileShape {
    static constexpr int kWaves = NW;
    static constexpr int kThreads = 64 * NW;
    static constexpr int kWM = BM / (16 * WMI);            // waves along rows
    static constexpr int kWN = NW / kWM;                   // waves along weight rows
    static_assert(kWM * kWN == NW && BW == kWN * 128, "waves of 64 x 128");
    static constexpr int kRows = BM + BW;
    static constexpr int kLoads = kRows / (8 * NW);        // 8-row loads per wave per stage
    static constexpr int kScBytes = MODE == 1 ? kRows * kScRow : 0;
    static constexpr int kBuf = kRows * kRowBytes + kScBytes;
    static constexpr int kGroupM = BM == 256 ? 4 : 8;      // row blocks per tile group
    static constexpr int kGroupN = 32 / kGroupM;           // weight tiles per tile group
};

__device__ __forceinline__ float silu_mul(float g, float u) {
    // g / (1 + e^-g): for very negative g, e^-g overflows to +inf and the
    // reciprocal gives 0, so the result is a signed zero, never NaN.
    const float e = __expf(-g);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// byte offset of 16-byte chunk c of tile row r inside a stage buffer
__device__ __forceinline__ int lds_chunk(int r, int c) {
    const int f = ((r >> 1) ^ ((r & 1) << 2)) & 7;
    return r * kRowBytes + ((c ^ f) & 7) * 16;
}

// Workgroup barrier that waits for this wave's LDS accesses only, not for
// the global loads of the next stage in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int MODE, int STAGE, int BM, int BW, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_tile(GemmParams p) {
    using TS = TileShape<MODE, BM, BW, NW>;
    constexpr int kWaves = TS::kWaves, kThreads = TS::kThreads;
    constexpr int kLoads = TS::kLoads, BUF = TS::kBuf;
    constexpr int kWN = TS::kWN;
    __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wm = w / kWN, wn = w % kWN;
    const int r16 = lane & 15, kg = lane >> 4;

    // ---- tile mapping
    constexpr int tile_cols = STAGE == 1 ? BW / 2 : BW;
    const int n_tiles = p.N / tile_cols;
    const uint32_t Lg = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t per_group = TS::kGroupM * TS::kGroupN;
    const uint32_t m_groups = (uint32_t)(p.max_mblocks + TS::kGroupM - 1) / TS::kGroupM;
    const uint32_t grp = Lg / per_group, r = Lg % per_group;
    const int mb = (int)((grp % m_groups) * TS::kGroupM + r % TS::kGroupM);
    const int nt = (int)((grp / m_groups) * TS::kGroupN + r / TS::kGroupM);
    if (nt >= n_tiles || mb >= p.max_mblocks) return;
    const int n_blocks = *p.n_padded / BM;
    if (mb >= n_blocks) return;
    const int e = p.block_expert[mb];
    const int row0 = mb * BM;
    const int n0 = nt * tile_cols;

    // ---- source rows: load i of wave w covers tile rows 8 (w + 8 i) .. +8;
    // this lane reads row 8 (w + 4 i) + lane / 8, bytes 16 (lane % 8) .. +16
    // of the stage. Tile rows [0, BM) are A rows, [BM, BM + BW) weight rows.
    const int lrow = lane >> 3, lchunk = lane & 7;
    auto a_row_of = [&](int row) -> int64_t {
        if (STAGE == 1) {
            const int a = p.sorted[row];
            return a < p.A ? (int64_t)((unsigned)a / (unsigned)p.k) : 0;
        }
        // a padding row re-reads the block's first row instead of an h row
        // nobody wrote
        return p.sorted[row] < p.A ? row : row0;
    };
    constexpr int EB = MODE == 0 ? 2 : 1;   // bytes per stride unit
    // Whether load i reads A or gate/up rows is the same for the whole wave,
    // so each load has a wave-uniform base and a 32-bit per-lane offset (the
    // host keeps every operand offset below 2^31 bytes). Its LDS destination
    // is dst + 8 KB * i: 64 tile rows further, same swizzle.
    const char* ld_base[kLoads];
    uint32_t ld_off[kLoads];
    const int dst = lds_chunk(8 * w + lrow, lchunk);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int t = 8 * (w + kWaves * i) + lrow;   // tile row
        if (8 * (w + kWaves * i) < BM) {
            ld_base[i] = reinterpret_cast<const char*>(p.a);
            ld_off[i] = (uint32_t)(a_row_of(row0 + t) * p.a_row * EB);
        } else {
            const int R = t - BM;
            const bool second = STAGE == 1 && 8 * (w + kWaves * i) - BM >= BW / 2;
            const int wrow = n0 + (STAGE == 1 ? R % (BW / 2) : R);
            ld_base[i] = reinterpret_cast<const char*>(second ? p.b1 : p.b0) + (int64_t)e * (second ? p.b1_e : p.b0_e) * EB;
            ld_off[i] = (uint32_t)((int64_t)wrow * (second ? p.b1_r : p.b0_r) * EB);
        }
        ld_off[i] += lchunk * 16;
    }
    // MXFP4: thread t stages the 8 scale bytes per stage of tile rows t,
    // t + 512, ...; a thread past the last tile row re-reads that row and
    // does not store it
    constexpr int kScLoads = MODE == 1 ? (TS::kRows + kThreads - 1) / kThreads : 0;
    const uint8_t* sc_src[kScLoads > 0 ? kScLoads : 1];
    if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < kScLoads; ++j) {
            const int t = min((int)threadIdx.x + kThreads * j, TS::kRows - 1);
            if (t < BM) {
                sc_src[j] = p.a_sc + a_row_of(row0 + t) * p.a_sc_row;
            } else {
                const int R = t - BM;
                const bool second = STAGE == 1 && R >= BW / 2;
                const int wrow = n0 + (STAGE == 1 ? R % (BW / 2) : R);
                const uint8_t* sb = second ? p.b1_sc : p.b0_sc;
                sc_src[j] =
                    sb + (int64_t)e * (second ? p.b1sc_e : p.b0sc_e) + (int64_t)wrow * (second ? p.b1sc_r : p.b0sc_r);
            }
        }
    }

    const int S = p.K / (MODE == 0 ? 64 : 256);   // stages; the host keeps it even

    // ---- global -> registers -> LDS
    i32x4_t st[kLoads];
    uint2 sc[kScLoads > 0 ? kScLoads : 1];
    auto issue = [&](int s) {
        s = s < S ? s : S - 1;    // past the end: re-read the last stage (L2 hit)
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            st[i] = *reinterpret_cast<const i32x4_t*>(ld_base[i] + (ld_off[i] + (uint32_t)(s * kRowBytes)));
        if constexpr (MODE == 1) {
#pragma unroll
            for (int j = 0; j < kScLoads; ++j) sc[j] = *reinterpret_cast<const uint2*>(sc_src[j] + s * kScRow);
        }
    };
    // scales go to LDS as [row][k-group][k-step] so that a lane's two bytes
    // of a stage are adjacent
    auto interleave = [](uint32_t d0, uint32_t d1, int hi) -> uint32_t {
        const uint32_t x = hi ? d0 >> 16 : d0, y = hi ? d1 >> 16 : d1;
        return (x & 0xffu) | ((y & 0xffu) << 8) | ((x & 0xff00u) << 8) | ((y & 0xff00u) << 16);
    };
    auto commit = [&](int b) {
        char* buf = lds + b * BUF;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) *reinterpret_cast<i32x4_t*>(buf + dst + i * 8 * kWaves * kRowBytes) = st[i];
        if constexpr (MODE == 1) {
            char* scb = buf + TS::kRows * kRowBytes;
#pragma unroll
            for (int j = 0; j < kScLoads; ++j) {
                const int t = threadIdx.x + kThreads * j;
                if (t < TS::kRows)
                    *reinterpret_cast<uint2*>(scb + t * kScRow) =
                        make_uint2(interleave(sc[j].x, sc[j].y, 0), interleave(sc[j].x, sc[j].y, 1));
            }
        }
    };

    // ---- MFMA over one LDS stage: wave (wm, wn) multiplies tile rows
    // wm*16*WMI .. +16*WMI by its 8 weight row blocks
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
    // fragment row block rb of a k-step: row 16 rb + r16, chunk 4 sub + kg
    const int rd0 = lds_chunk(r16, kg), rd1 = lds_chunk(r16, 4 + kg);
    auto compute = [&](int b) {
        const char* buf = lds + b * BUF;
        uint32_t as[WMI], bs[8];
        if constexpr (MODE == 1) {
            const char* scb = buf + TS::kRows * kRowBytes;
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi)
                as[mi] = *reinterpret_cast<const uint16_t*>(scb + ((wm * WMI + mi) * 16 + r16) * kScRow + kg * 2);
#pragma unroll
            for (int ni = 0; ni < 8; ++ni)
                bs[ni] = *reinterpret_cast<const uint16_t*>(scb + (BM + b_rb(ni) * 16 + r16) * kScRow + kg * 2);
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int rd = sub ? rd1 : rd0;
            i32x4_t af[WMI], bf[8];
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi)
                af[mi] = *reinterpret_cast<const i32x4_t*>(buf + (wm * WMI + mi) * 16 * kRowBytes + rd);
#pragma unroll
            for (int ni = 0; ni < 8; ++ni)
                bf[ni] = *reinterpret_cast<const i32x4_t*>(buf + (BM + b_rb(ni) * 16) * kRowBytes + rd);
#pragma unroll
            for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
                for (int ni = 0; ni < 8; ++ni) {
                    if constexpr (MODE == 0) {
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, af[mi]), __builtin_bit_cast(bf16x8_t, bf[ni]), acc[mi][ni],
                            0, 0, 0);
                    } else {
                        const i32x8_t a8 = {af[mi][0], af[mi][1], af[mi][2], af[mi][3], 0, 0, 0, 0};
                        const i32x8_t b8 = {bf[ni][0], bf[ni][1], bf[ni][2], bf[ni][3], 0, 0, 0, 0};
                        // the byte of the scale words for this k-step: op_sel
                        if (sub == 0)
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                a8, b8, acc[mi][ni], 4, 4, 0, (int)as[mi], 0, (int)bs[ni]);
                        else
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                a8, b8, acc[mi][ni], 4, 4, 1, (int)as[mi], 1, (int)bs[ni]);
                    }
                }
            // MXFP4 holds one k-step of fragments at a time (register budget)
            if constexpr (MODE == 1) __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- pipeline: stage s is multiplied from buffer s % 2 while the loads
    // of stage s + 1 are in flight
    issue(0);
    commit(0);
    lds_barrier();
    for (int s = 0; s < S; s += 2) {
        issue(s + 1);
        compute(0);
        commit(1);
        lds_barrier();
        issue(s + 2);
        compute(1);
        commit(0);
        lds_barrier();
    }

    // ---- epilogues: acc[mi][ni][i] is row wm*16*WMI + mi*16 + kg*4 + i,
    // column r16 of the ni-th column block
    if constexpr (STAGE == 1 && MODE == 0) {
        uint16_t* h = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 64 + j * 16 + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t row = row0 + wm * 16 * WMI + mi * 16 + kg * 4 + i;
                    h[row * p.N + col] = f32_to_bf16_bits(silu_mul(acc[mi][j][i], acc[mi][4 + j][i]));
                }
            }
    } else if constexpr (STAGE == 1 && MODE == 1) {
        uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c0 = n0 + wn * 64 + q * 32;   // first of the 32 h columns of this scale group
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float h0 = silu_mul(acc[mi][2 * q][i], acc[mi][4 + 2 * q][i]);
                    const float h1 = silu_mul(acc[mi][2 * q + 1][i], acc[mi][4 + 2 * q + 1][i]);
                    const uint32_t b0 = __float_as_uint(h0), b1 = __float_as_uint(h1);
                    uint32_t amax = max(b0 & 0x7fffffffu, b1 & 0x7fffffffu);
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
                    const int sx = group_exponent(amax);
                    const E2m1Thresholds th = e2m1_thresholds(sx);
                    const uint32_t k0 = e2m1_code(b0, th), k1 = e2m1_code(b1, th);
                    const uint32_t o0 = (uint32_t)__shfl_xor((int)k0, 1), o1 = (uint32_t)__shfl_xor((int)k1, 1);
                    const int64_t row = row0 + wm * 16 * WMI + mi * 16 + kg * 4 + i;
                    uint8_t* rp = hq + row * (p.N / 2);
                    if ((r16 & 1) == 0) {
                        rp[(c0 + r16) / 2] = (uint8_t)(k0 | (o0 << 4));
                        rp[(c0 + 16 + r16) / 2] = (uint8_t)(k1 | (o1 << 4));
                    }
                    if (r16 == 0) p.out_sc[row * (p.N / 32) + c0 / 32] = (uint8_t)(sx + 127);
                }
            }
    } else {
        float* y = reinterpret_cast<float*>(p.out);
#pragma unroll
        for (int mi = 0; mi < WMI; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = p.sorted[row0 + wm * 16 * WMI + mi * 16 + kg * 4 + i];
                if (a >= p.A) continue;
                float* yr = y + (int64_t)a * p.N + n0 + wn * 128 + r16;
#pragma unroll
                for (int ni = 0; ni < 8; ++ni) yr[ni * 16] = acc[mi][ni][i];
            }
    }
}

template <int MODE, int STAGE, int BM, int BW, int NW>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
    using TS = TileShape<MODE, BM, BW, NW>;
    const int64_t n_tiles = p.N / (STAGE == 1 ? BW / 2 : BW);
    const int64_t m_groups = (p.max_mblocks + TS::kGroupM - 1) / TS::kGroupM;
    const int64_t n_groups = (n_tiles + TS::kGroupN - 1) / TS::kGroupN;
    const int64_t grid = m_groups * n_groups * TS::kGroupM * TS::kGroupN;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_tile<MODE, STAGE, BM, BW, NW>), dim3((unsigned)grid), dim3(TS::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Tile shapes: 0 = 256 x 256 (eight waves; MXFP4: 128 x 256, four waves of
// one per SIMD, whose accumulators fit only in the larger register budget),
// 1 = 128 x 512 (bf16, eight waves).
int gemm_tile_rows(int mode, int shape) { return shape == 0 && mode == 0 ? 256 : 128; }

int gemm_tile_cols(int shape, int stage) {
    const int bw = shape == 1 ? 512 : 256;
    return stage == 1 ? bw / 2 : bw;
}

int gemm_tile_k_granule(int mode) { return mode == 0 ? 2 * 64 : 2 * 256; }

bool gemm_tile_supported(int mode, int shape) { return shape == 0 || (shape == 1 && mode == 0); }

hipError_t launch_gemm_tile(int mode, int shape, int stage, const GemmParams& p, hipStream_t s) {
    if (!gemm_tile_supported(mode, shape) || p.N % gemm_tile_cols(shape, stage) != 0 ||
        p.K % gemm_tile_k_granule(mode) != 0)
        return hipErrorInvalidValue;
    if (mode == 1) return stage == 1 ? launch_one<1, 1, 128, 256, 4>(p, s) : launch_one<1, 2, 128, 256, 4>(p, s);
    if (shape == 0) return stage == 1 ? launch_one<0, 1, 256, 256, 8>(p, s) : launch_one<0, 2, 256, 256, 8>(p, s);
    return stage == 1 ? launch_one<0, 1, 128, 512, 8>(p, s) : launch_one<0, 2, 128, 512, 8>(p, s);
}

}  // namespace moe
