// MXFP4 gemm2 with K = 512 (the TP2 shard's inter_dim) for many tokens per
// expert: a workgroup keeps one sorted block of h rows in registers and walks
// the output columns in tiles of 128 weight rows (ROCm/aiter PR "TP2 MXFP4
// fused-MoE configs for Qwen3.5-397B", Details: inter_dim 512 and the large
// token buckets).
//
// With K = 512 a row of h is 256 bytes of e2m1 codes plus 16 scale bytes, so
// a block of 256 rows fits in the registers of eight waves (64 per wave, 64
// VGPRs of fragments each). The weight tiles of the block's expert then
// stream through LDS, four buffers deep, each used by all eight waves: the
// LDS-tiled kernel instead loaded a whole K of both operands for every
// 256 x 256 output tile, with the next tile's first loads waiting behind the
// epilogue. Here the loads of tile j + 3 are in flight while tile j is
// multiplied and its y rows stored, and h is read once per block instead of
// once per output tile.
//
// Every output element is the same chain of four 16x16x128 block-scaled
// MFMAs over K in ascending order, with the weight fragment as the first
// operand, as in the other MXFP4 kernels: the results are bit-identical.
//
// y rows (bf16, RNE) go out with buffer stores; a padding row's lanes get an
// offset past the buffer's end, which the hardware drops. Every wave thus
// issues the same number of vector memory instructions per tile, so the
// s_waitcnt counts that keep three weight tiles in flight stay exact (stores
// count in the same counter as loads).
//
// LDS layout: a 256-byte code row is 16 chunks of 16 bytes; chunk c of row r
// sits at position c ^ (r % 16), so the 16 rows of one MFMA fragment (same
// chunk) hit 16 different 16-byte bank groups. The loads fetch for each lane
// the chunk the swizzle stores at that lane's position.
#include <utility>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRowB = 256;            // code bytes of one K = 512 row
constexpr int kScB = 16;              // scale bytes of one row
constexpr int kBN = 128;              // weight rows (output columns) per tile
constexpr int kNW = 8;                // waves per workgroup
constexpr int kNBuf = 4;              // weight tile buffers
constexpr int kTileCodes = kBN * kRowB;            // 32 KB
constexpr int kBufB = kTileCodes + kBN * kScB;     // 34 KB per buffer
constexpr int kLdsB = kNBuf * kBufB;               // 136 KB
// per wave per weight tile: 4 code loads (16 B per lane) + 1 scale load (4 B)
constexpr int kLB = kBN * kRowB / 1024 / kNW + kBN * kScB / 256 / kNW;
static_assert(kLB == 5, "load count per tile");

template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// s_waitcnt vmcnt(n) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// byte kg of each of the four dwords, packed: byte u of the result is the
// scale of k-step u for this lane's k-group
__device__ __forceinline__ uint32_t pack_scales(i32x4_t v, int kg) {
    const int sh = 8 * kg;
    return (((uint32_t)v[0] >> sh) & 0xffu) | ((((uint32_t)v[1] >> sh) & 0xffu) << 8) |
           ((((uint32_t)v[2] >> sh) & 0xffu) << 16) | ((((uint32_t)v[3] >> sh) & 0xffu) << 24);
}

// BM = 256 or 128 rows; waves: BM / 64 along rows, the rest along the 128
// columns of a tile (NBW 16-column blocks each)
template <int BM>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm2_rows_kernel(GemmParams p, int nsplit) {
    constexpr int kWM = BM / 64, kWN = kNW / kWM, NBW = kBN / kWN / 16;
    // y stores per wave per tile (one 8-byte store per row group and column block)
    constexpr int kS = 4 * NBW;
    static_assert(2 * kLB + 3 * kS < 64, "waits fit vmcnt");
    __shared__ __attribute__((aligned(16))) char lds[kLdsB];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w / kWN, wn = w % kWN;
    const int r16 = lane & 15, kg = lane >> 4;

    // ---- workgroup -> (row block, column range); eight equal contiguous
    // ranges of the real blocks, one per XCD (workgroup b runs on XCD b % 8)
    const int n_blocks = __builtin_amdgcn_readfirstlane(*p.n_padded) / BM;
    const uint32_t total = (uint32_t)n_blocks * (uint32_t)nsplit;
    const uint32_t per_xcd = (total + 7u) / 8u;
    const uint32_t xcd = blockIdx.x & 7u, jj = blockIdx.x >> 3;
    if (jj >= per_xcd) return;
    const uint32_t L = xcd * per_xcd + jj;
    if (L >= total) return;
    const int mb = (int)(L % (uint32_t)n_blocks), ns = (int)(L / (uint32_t)n_blocks);
    const int e = __builtin_amdgcn_readfirstlane(p.block_expert[mb]);
    const int row0 = mb * BM;
    const int ntiles = p.N / kBN / nsplit;
    const int col_base = ns * ntiles * kBN;
    // the y row offsets of this lane's rows wm * 64 + mi * 16 + r16 (a
    // padding row gets an offset past the buffer, so its stores are
    // dropped), taken before any load to LDS is issued: a wait for a plain
    // load issued among those would wait for all of them
    uint32_t y_off[4];
    const uint32_t y_stride = (uint32_t)(p.out_row * 2);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int a = p.sorted[row0 + wm * 64 + mi * 16 + r16];
        y_off[mi] = a < p.A ? (uint32_t)a * y_stride : 0xFFFFFFF0u;
    }

    // ---- loads. A (h rows by flat assignment; a padding row reads row 0)
    // into the region of buffers 2 and 3, weight tiles into buffer j % 4.
    const uint8_t* h = reinterpret_cast<const uint8_t*>(p.a);
    auto a_row_of = [&](int row) -> int64_t {
        const int a = p.sorted[row];
        return a < p.A ? (int64_t)a : 0;
    };
    char* const a_lds = lds + 2 * kBufB;
    constexpr int kALoads = BM / 4 / kNW;           // 16-byte loads per wave (4 rows each)
    constexpr int kAScLoads = BM * kScB / 256 / kNW;  // 4-byte loads per wave (64 dwords each)
    static_assert(kALoads * 4 * kNW == BM && kAScLoads * 256 * kNW == BM * kScB, "whole A loads");
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
        const int blk = w + kNW * i;                 // 1 KB LDS block: rows 4 blk .. +3
        const int r = 4 * blk + (lane >> 4), pos = lane & 15;
        const int c = pos ^ (r & 15);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(h + a_row_of(row0 + r) * p.a_row + c * 16),
            (lds_ptr_t)(a_lds + blk * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAScLoads; ++i) {
        const int d = (w + kNW * i) * 64 + lane;     // dword of the [BM, 16] scale block
        const int r = d >> 2;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(p.a_sc + a_row_of(row0 + r) * p.a_sc_row + (d & 3) * 4),
            (lds_ptr_t)(a_lds + BM * kRowB + (w + kNW * i) * 256), 4, 0, 0);
    }
    // weight tile j: rows col_base + j * 128 + r of w2_e (clamped: past the
    // last tile the last one is loaded again, into a buffer nobody reads)
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(p.b0) + (int64_t)e * p.b0_e;
    const uint8_t* sbase = p.b0_sc + (int64_t)e * p.b0sc_e;
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int blk = w + kNW * i;
        const int r = 4 * blk + (lane >> 4), pos = lane & 15;
        b_off[i] = (uint32_t)((int64_t)r * p.b0_r + ((pos ^ (r & 15)) * 16));
    }
    const int sd = w * 64 + lane;                    // dword of the [128, 16] scale tile
    const uint32_t s_off = (uint32_t)((int64_t)(sd >> 2) * p.b0sc_r + (sd & 3) * 4);
    auto load_tile = [&](int j) {
        j = j < ntiles ? j : ntiles - 1;
        char* buf = lds + (j & 3) * kBufB;
        const int64_t n0 = col_base + (int64_t)j * kBN;
        const uint8_t* wt = wbase + n0 * p.b0_r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(wt + b_off[i]),
                                             (lds_ptr_t)(buf + (w + kNW * i) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sbase + n0 * p.b0sc_r + s_off),
                                         (lds_ptr_t)(buf + kTileCodes + w * 256), 4, 0, 0);
    };
    load_tile(0);
    load_tile(1);

    // ---- this wave's h fragments and scales into registers: rows
    // wm * 64 + mi * 16 + r16, k-step u = chunks 4u .. 4u + 3 (lane kg)
    wait_vm_lgkm<2 * kLB>();
    barrier();
    i32x4_t af[4][4];
    uint32_t asc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + mi * 16 + r16;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            af[mi][u] = *reinterpret_cast<const i32x4_t*>(a_lds + r * kRowB + (((4 * u + kg) ^ r16) * 16));
        asc[mi] = pack_scales(*reinterpret_cast<const i32x4_t*>(a_lds + BM * kRowB + r * kScB), kg);
    }
    // every wave is past its A reads before buffers 2 and 3 are refilled
    wait_vm_lgkm<2 * kLB>();
    barrier();
    load_tile(2);

    // y as a buffer resource: stores at an offset past num_records are dropped
    const uint32_t y_bytes = (uint32_t)((int64_t)p.A * p.out_row * 2);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(p.out, (short)0, (int)y_bytes, 0x00020000);

    f32x4_t acc[4][NBW];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mi][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < ntiles; ++j) {
        // tile j landed for every wave; every wave is done with tile j - 1
        // (loads issued after tile j's: tiles j + 1, j + 2 and the y stores
        // of up to three earlier tiles)
        if (j >= 3)
            wait_vm_lgkm<2 * kLB + 3 * kS>();
        else if (j == 2)
            wait_vm_lgkm<2 * kLB + 2 * kS>();
        else if (j == 1)
            wait_vm_lgkm<2 * kLB + kS>();
        else
            wait_vm_lgkm<2 * kLB>();
        barrier();
        load_tile(j + 3);
        const char* buf = lds + (j & 3) * kBufB;
        // weight scales of the wave's column blocks, packed per k-step
        uint32_t bsc[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int r = (wn * NBW + nb) * 16 + r16;
            bsc[nb] = pack_scales(*reinterpret_cast<const i32x4_t*>(buf + kTileCodes + r * kScB), kg);
        }
        static_for<4>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            i32x4_t bf[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int r = (wn * NBW + nb) * 16 + r16;
                bf[nb] = *reinterpret_cast<const i32x4_t*>(buf + r * kRowB + (((4 * u + kg) ^ r16) * 16));
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const i32x8_t a8 = {af[mi][u][0], af[mi][u][1], af[mi][u][2], af[mi][u][3], 0, 0, 0, 0};
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const i32x8_t b8 = {bf[nb][0], bf[nb][1], bf[nb][2], bf[nb][3], 0, 0, 0, 0};
                    acc[mi][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        b8, a8, acc[mi][nb], 4, 4, u, (int)bsc[nb], u, (int)asc[mi]);
                }
            }
        });
        // y: lane holds columns 4 kg .. +3 of column block nb for row r16
        const uint32_t col_b = (uint32_t)(col_base + j * kBN + wn * NBW * 16 + kg * 4) * 2;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const u32x2_t pk = {
                    bf16x2_bits(acc[mi][nb][0], acc[mi][nb][1]),
                    bf16x2_bits(acc[mi][nb][2], acc[mi][nb][3])};
                const uint32_t off = y_off[mi] == 0xFFFFFFF0u ? 0xFFFFFFF0u : y_off[mi] + col_b + nb * 32;
                __builtin_amdgcn_raw_buffer_store_b64(pk, yr, off, 0, 0);
            }
        // zeroed through registers the compiler cannot see as constants, so
        // the next tile's first MFMAs accumulate in place
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                float z;
                __asm__("v_mov_b32 %0, 0" : "=v"(z));
                acc[mi][nb] = f32x4_t{z, z, z, z};
            }
    }
    // drain the loads past the end before the workgroup's LDS is released
    wait_vm_lgkm<0>();
}

template <int BM>
hipError_t launch_rows(const GemmParams& p, int nsplit, hipStream_t s) {
    const int64_t grid = ((int64_t)p.max_mblocks * nsplit + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm2_rows_kernel<BM>, dim3((unsigned)grid), dim3(64 * kNW), 0, s, p, nsplit);
    return hipGetLastError();
}

}  // namespace

bool gemm2_rows_supported(int64_t K, int64_t N, int64_t A, int64_t out_row) {
    return K == 512 && N % kBN == 0 && (int64_t)A * out_row * 2 < (int64_t)0xFFFFFFF0;
}

// Column ranges per row block: enough workgroups to fill the chip a few times
int gemm2_rows_split(int bm, int64_t max_mblocks, int64_t N) {
    int s = 1;
    while (s < 8 && max_mblocks * s < 1024 && (N / kBN) % (2 * s) == 0) s *= 2;
    (void)bm;
    return s;
}

hipError_t launch_gemm2_rows(int bm, const GemmParams& p, hipStream_t s) {
    if (p.K != 512 || p.N % kBN != 0) return hipErrorInvalidValue;
    const int nsplit = gemm2_rows_split(bm, p.max_mblocks, p.N);
    if (bm == 256) return launch_rows<256>(p, nsplit, s);
    if (bm == 128) return launch_rows<128>(p, nsplit, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
