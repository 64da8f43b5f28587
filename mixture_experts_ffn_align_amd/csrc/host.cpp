// Host side of libmoeffn: argument checks, configuration choice, workspace
// layout and the launch sequence behind the C ABI declared in moeffn.h.
//
// Every check runs before the first launch, so a call that fails has
// enqueued nothing (Liger-Kernel PR #1377, Testing Done: mismatched gate
// hidden dims fail before any descriptor is built; strided grad inputs are
// rejected before any native allocation). A layout the kernels cannot read
// is rejected, never read as if contiguous (LightLLM issue #1467).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "gemm_persist.h"
#include "moe_internal.h"
#include "prep.h"
#include "moeffn.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MOE_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

const char* dtype_name(int d) {
    switch (d) {
        case MOE_DT_BF16: return "bf16";
        case MOE_DT_F32: return "f32";
        case MOE_DT_I32: return "i32";
        case MOE_DT_FP4X2: return "fp4x2";
        case MOE_DT_E8M0: return "e8m0";
        default: return "?";
    }
}

int elem_bytes(int d) {
    switch (d) {
        case MOE_DT_BF16: return 2;
        case MOE_DT_F32: case MOE_DT_I32: return 4;
        case MOE_DT_FP4X2: case MOE_DT_E8M0: return 1;
        default: return 0;
    }
}

int64_t numel(const moe_tensor_t& t) {
    int64_t n = 1;
    for (int i = 0; i < t.ndim; ++i) n *= t.size[i];
    return n;
}

// Basic descriptor sanity: dtype, rank, non-negative sizes, positive strides
// on dimensions longer than 1, and data present when the tensor is not empty.
int check_desc(const moe_tensor_t* t, const char* name, int dtype, int ndim) {
    if (!t) return fail(MOE_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->dtype != dtype)
        return fail(MOE_ERR_DTYPE, "%s: dtype %s, expected %s", name, dtype_name(t->dtype), dtype_name(dtype));
    if (t->ndim != ndim) return fail(MOE_ERR_SHAPE, "%s: %d dims, expected %d", name, t->ndim, ndim);
    for (int i = 0; i < ndim; ++i) {
        if (t->size[i] < 0) return fail(MOE_ERR_SHAPE, "%s: negative size in dim %d", name, i);
        if (t->size[i] > 1 && t->stride[i] <= 0)
            return fail(MOE_ERR_LAYOUT, "%s: stride %lld in dim %d must be positive", name,
                        (long long)t->stride[i], i);
    }
    if (numel(*t) > 0 && !t->data) return fail(MOE_ERR_NULL, "%s: data is NULL", name);
    return MOE_OK;
}

int check_shape(const moe_tensor_t& t, const char* name, std::initializer_list<int64_t> want) {
    int i = 0;
    for (int64_t w : want) {
        if (t.size[i] != w) {
            return fail(MOE_ERR_SHAPE, "%s: size[%d] = %lld, expected %lld", name, i, (long long)t.size[i],
                        (long long)w);
        }
        ++i;
    }
    return MOE_OK;
}

// Byte range [lo, hi) a strided tensor can touch.
void extent(const moe_tensor_t& t, uintptr_t* lo, uintptr_t* hi) {
    int64_t span = 0;
    for (int i = 0; i < t.ndim; ++i)
        if (t.size[i] > 0) span += (t.size[i] - 1) * t.stride[i];
    *lo = (uintptr_t)t.data;
    *hi = *lo + (uintptr_t)((span + 1) * elem_bytes(t.dtype));
}

bool overlaps(const moe_tensor_t& a, const moe_tensor_t& b) {
    if (numel(a) == 0 || numel(b) == 0 || !a.data || !b.data) return false;
    uintptr_t al, ah, bl, bh;
    extent(a, &al, &ah);
    extent(b, &bl, &bh);
    return al < bh && bl < ah;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Two 3-D views of one buffer whose element sets are disjoint although their
// byte ranges interleave: same sizes and strides, rows that do not overlap
// (row stride >= row length, last stride 1), and one view shifted from the
// other by whole rows inside an expert block of P = stride(0) / stride(1)
// rows, with the shifted rows staying clear of the other view's rows modulo
// P. Packed halves w[:, :I] and w[:, I:] of [E, 2I, H] are the case meant.
bool interleaved_disjoint(const moe_tensor_t& a, const moe_tensor_t& b) {
    if (a.ndim != 3 || b.ndim != 3 || a.dtype != b.dtype) return false;
    for (int i = 0; i < 3; ++i)
        if (a.size[i] != b.size[i] || a.stride[i] != b.stride[i]) return false;
    const int64_t s0 = a.stride[0], s1 = a.stride[1], eb = elem_bytes(a.dtype);
    if (a.stride[2] != 1 || s1 < a.size[2] || s1 <= 0 || s0 <= 0 || s0 % s1 != 0) return false;
    const int64_t diff = (int64_t)((uintptr_t)b.data - (uintptr_t)a.data);
    const int64_t d = diff < 0 ? -diff : diff;
    if (d % (eb * s1) != 0) return false;
    const int64_t dr = d / (eb * s1), P = s0 / s1, rows = a.size[1];
    return dr < P && dr >= rows && dr + rows <= P;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t align_capacity(int64_t A, int64_t E, int64_t bm) {
    if (A <= 0) return 0;
    int64_t cap = A + std::min(E, A) * (bm - 1);
    return (cap + bm - 1) / bm * bm;
}

bool valid_bm(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// -------------------------------------------------------- configurations
//
// The list of tile configurations the fused forward can run. The choice
// depends only on (mode, T, H, I, E, k), never on strides or addresses, so
// strided and contiguous calls execute the same arithmetic. Entries are only
// ever appended: the tuned table and force_config refer to them by index.
struct Cfg {
    int bm, wk1, wk2, nb;
    int tile;     // 0: weight-streaming GEMMs; 1 + shape: LDS-tiled GEMMs of that tile shape
    int g2;       // -1, or the entry whose gemm2 kernel runs gemm2 (own block size and align)
    int nt2 = 1;  // MXFP4 gemm2 on the stream with K = 512: 256-column tiles per workgroup
    int fuse = 0; // 1: gemm2 and the combine in one kernel, per token (few tokens; MXFP4 K = 512, bf16
                  // K split 4); 2: besides, gemm1 per slot without the align (expert from the ids)
    int persist = 0;  // MXFP4 gemm1 on the persistent weight stream with this many waves (4 or 8)
    int persist2 = 0; // 1: MXFP4 gemm2 (K = 512) on the persistent weight stream
};
const Cfg kConfigs[] = {
    {16, 4, 4, 4, 0, -1}, {32, 4, 4, 4, 0, -1}, {64, 2, 2, 4, 0, -1},
    {16, 2, 2, 4, 0, -1}, {32, 2, 2, 4, 0, -1}, {64, 1, 1, 4, 0, -1},
    {16, 1, 1, 4, 0, -1}, {32, 1, 1, 4, 0, -1}, {128, 1, 1, 4, 0, -1},
    {32, 1, 1, 2, 0, -1}, {64, 1, 1, 2, 0, -1},    // bf16 only: narrow waves, deep weight ring
    {256, 1, 1, 4, 1, -1}, {128, 1, 1, 4, 2, -1},  // many rows per expert: weight reuse
    {64, 1, 1, 4, 3, -1}, {32, 1, 1, 4, 4, -1},    // LDS-staged weight stream
    {64, 1, 1, 4, 5, -1},
    // gemm1 on the register stream, gemm2 on an LDS-staged tile
    {16, 1, 1, 4, 0, 15}, {16, 2, 2, 4, 0, 15}, {16, 4, 4, 4, 0, 15},
    {16, 1, 1, 4, 0, 14}, {16, 2, 2, 4, 0, 14}, {16, 4, 4, 4, 0, 14},
    {64, 1, 1, 4, 0, 13},
    // MXFP4, K = 512: gemm2 workgroups take 2, 4 or 8 column tiles of a row block
    {16, 1, 1, 4, 0, -1, 2}, {16, 1, 1, 4, 0, -1, 4}, {16, 1, 1, 4, 0, -1, 8},
    {32, 1, 1, 4, 0, -1, 4}, {16, 4, 1, 4, 0, -1, 2}, {16, 2, 1, 4, 0, -1, 2},
    {16, 2, 1, 4, 0, -1, 4}, {32, 1, 1, 4, 0, -1, 8},
    // the same with 64-row blocks (mid T)
    {64, 1, 1, 4, 0, -1, 2}, {64, 1, 1, 4, 0, -1, 4}, {64, 1, 1, 4, 0, -1, 8},
    // MXFP4, K = 512, few tokens: gemm1 on the stream, gemm2 fused with the combine
    {16, 1, 1, 4, 0, -1, 1, 1}, {16, 2, 1, 4, 0, -1, 1, 1}, {16, 4, 1, 4, 0, -1, 1, 1},
    // the same with gemm1 per slot (K split 4) and no align
    {16, 4, 1, 4, 0, -1, 1, 2},
    // 128 x 256 tiles (about 64 to 160 rows per expert); gemm2 on them, on
    // the MXFP4 multi-tile stream with 64-row blocks, or on 256 x 256 tiles
    {128, 1, 1, 4, 6, -1}, {128, 1, 1, 4, 6, 31}, {128, 1, 1, 4, 6, 11},
    // MXFP4 with K = 512 in gemm2: gemm1 on 256 x 256 or 128 x 256 tiles,
    // gemm2 with its h rows in registers walking 128-column weight tiles
    // (entries 43 and 44 name that gemm2 kernel; as gemm1 they cannot run)
    {256, 1, 1, 4, 1, 43}, {128, 1, 1, 4, 6, 44},
    {256, 1, 1, 4, 7, -1}, {128, 1, 1, 4, 8, -1},
    // the same with the other block size for gemm2 (a second padded layout)
    {256, 1, 1, 4, 1, 44}, {128, 1, 1, 4, 6, 43},
    // MXFP4 256 x 256 with 128-byte gemm1 stages; gemm2 on its own tile, or
    // register-resident with 256 or 128 rows
    {256, 1, 1, 4, 9, -1}, {256, 1, 1, 4, 9, 43}, {256, 1, 1, 4, 9, 44},
    // MXFP4 128 x 256 with 128-byte stages; gemm2 on its own tile, or
    // register-resident with 128 or 256 rows
    {128, 1, 1, 4, 10, -1}, {128, 1, 1, 4, 10, 44}, {128, 1, 1, 4, 10, 43},
    // mid T (about 20 to 60 rows per expert): gemm1 on 64 x 512 tiles or on
    // the weight stream, gemm2 register-resident with 128-row blocks (its
    // own padded layout)
    {64, 1, 1, 4, 3, 44}, {32, 1, 1, 4, 0, 44}, {64, 1, 1, 4, 0, 44}, {16, 1, 1, 4, 0, 44},
    // MXFP4 gemm1 as a persistent weight stream (one workgroup per compute
    // unit, 4 or 8 waves), gemm2 on the multi-tile stream or register-resident
    {16, 1, 1, 4, 0, -1, 4, 0, 4}, {16, 1, 1, 4, 0, -1, 8, 0, 4}, {32, 1, 1, 4, 0, -1, 8, 0, 4},
    {16, 1, 1, 4, 0, -1, 4, 0, 8}, {16, 1, 1, 4, 0, -1, 8, 0, 8}, {32, 1, 1, 4, 0, -1, 8, 0, 8},
    {32, 1, 1, 4, 0, 44, 1, 0, 4}, {32, 1, 1, 4, 0, 44, 1, 0, 8},
    // both GEMMs on persistent weight streams (gemm2 with K = 512), or gemm2 only
    {16, 1, 1, 4, 0, -1, 1, 0, 4, 1}, {32, 1, 1, 4, 0, -1, 1, 0, 4, 1}, {16, 1, 1, 4, 0, -1, 1, 0, 8, 1},
    {32, 1, 1, 4, 0, -1, 1, 0, 8, 1}, {16, 1, 1, 4, 0, -1, 1, 0, 0, 1}, {32, 1, 1, 4, 0, -1, 1, 0, 0, 1},
    // the same with 64-row blocks (about 40 to 60 rows per expert)
    {64, 1, 1, 4, 0, -1, 1, 0, 4, 1}, {64, 1, 1, 4, 0, -1, 1, 0, 0, 1}, {64, 1, 1, 4, 0, 44, 1, 0, 4},
    // bf16 320 x 256 tiles (about 200 to 320 rows per expert: one block
    // each); gemm2 on them or on 256 x 256 tiles (a second padded layout)
    {320, 1, 1, 4, 11, -1}, {320, 1, 1, 4, 11, 11},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// Per-bucket choices measured by the tuner (mixture_experts_ffn_align_amd/
// tune.py): every valid config timed on the layer's synthetic inputs, the
// fastest one whose output passes the error gate against the built-in
// choice kept. Exact matches only; other shapes use the rules below.
struct TunedRow {
    int mode;
    int64_t H, I, E, E_local, k;
    int bucket;
    int config;
    float us;    // measured GPU time per call (reference only)
};
const TunedRow kTuned[] = {
#include "tuned_configs.inc"
    {-1, 0, 0, 0, 0, 0, 0, -1, 0.f},   // end
};

int bucket_of(int64_t T) {
    int b = 1;
    while (b < T && b < 32768) b <<= 1;
    return b;
}

// Index of the tiled config of a tile shape, or -1 when it cannot run
// these sizes.
int tile_config(int md, int shape, int64_t H, int64_t I) {
    if (!gemm_tile_supported(md, shape)) return -1;
    const int gran = gemm_tile_k_granule(md, shape);
    if (H % gran != 0 || I % gran != 0 || I % gemm_tile_cols(shape, 1) != 0 || H % gemm_tile_cols(shape, 2) != 0)
        return -1;
    for (int c = 0; c < kNumConfigs; ++c)
        if (kConfigs[c].tile == shape + 1) return c;
    return -1;
}

// Default configuration per token bucket, from measurements on MI355X
// (Qwen3-235B-shaped bf16 and the TP2 MXFP4 shard):
//  * enough rows per expert: LDS-tiled GEMMs (bf16: 64 x 256 tiles with
//    three stages in flight from 0.1 expected rows per expert, 128 x 512 from
//    64, 256 x 256 from 128, 320 x 256 where the typical busiest expert has
//    257 to 320 rows, so one block holds it; MXFP4: 64 x 512 from 64 rows,
//    256 x 256 from 128);
//  * otherwise the register weight stream, whose block rows cover the
//    typical busiest expert of the bucket in one block (each expert's
//    weights stream from HBM once) and whose K split grows only while the
//    grid would not fill the chip; its gemm2 moves to an LDS-staged tile
//    (own block size, second layout) where that measured faster, or, for
//    MXFP4 with I = 512, to workgroups that take 2-8 column tiles each.
// E counts the experts over all shards of an expert-parallel group and sets
// the rows per expert; E_local (the call's own experts) only moves a bf16
// shard with 64-128 rows per expert to 256 x 256 tiles when its 128 x 512
// grid would leave half the CUs idle. Tiles never split K, so the tile shape
// keeps the sums bit-identical to the unsharded call, and the register
// stream's K split is chosen from E alone.
// Compute units of the current device (256 if it cannot be asked).
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

// Whether a config's persistent weight streams (if any) can run this call:
// MXFP4, the kernels' K and N, and at most 256 items per compute unit.
bool persist_fits(const Cfg& c, int md, int64_t A, int64_t E, int64_t H, int64_t I) {
    if (!c.persist && !c.persist2) return true;
    if (md != 1) return false;
    const int64_t cap = (int64_t)device_cus() * 256;
    if (c.persist && (!gemm1_persist_supported(c.bm, c.persist, H, I) ||
                      align_capacity(A, E, c.bm) / c.bm * (I / (32 * c.persist)) > cap))
        return false;
    if (c.persist2 && (!gemm2_persist_supported(c.bm, I, H) || align_capacity(A, E, c.bm) / c.bm * (H / 256) > cap))
        return false;
    return true;
}

int heuristic_config(int mode, int64_t T, int64_t H, int64_t I, int64_t E, int64_t E_local, int64_t k,
                     bool persist = true) {
    const int64_t bucket = bucket_of(T);
    const double rows = (double)bucket * (double)k / (double)E;   // expected rows per expert
    const double busy = rows + 3.0 * __builtin_sqrt(rows);          // typical maximum
    const int md = mode == MOE_MODE_MXFP4 ? 1 : 0;
    const int64_t experts = std::min<int64_t>(bucket * k, E);      // touched at most
    int c = -1;
    if (md == 0) {
        int shape = -1;
        if (rows >= 128.0) shape = busy > 256.0 && busy <= 320.0 ? 10 : 0;
        else if (rows >= 64.0) shape = 1;
        else if (rows >= 0.1) shape = 4;
        const int64_t grid1 = std::min<int64_t>(bucket * k, E_local) * (int64_t)std::ceil(rows / 128.0) *
                              (I / gemm_tile_cols(1, 1));
        if (shape == 1 && grid1 < 128 && tile_config(0, 0, H, I) >= 0) shape = 0;
        if (shape >= 0) c = tile_config(0, shape, H, I);
        if (c < 0 && shape == 10) c = tile_config(0, 0, H, I);
        if (c < 0 && shape >= 0 && shape != 4) c = tile_config(0, 4, H, I);
    } else {
        if (rows >= 128.0) c = tile_config(1, 0, H, I);
        else if (rows >= 64.0) c = tile_config(1, 2, H, I);
        // with K = 512 in gemm2 (I = 512), its h rows stay in registers
        if (c == tile_config(1, 0, H, I) && c >= 0 && I == 512) c = 41;
    }
    if (c >= 0) return c;
    // MXFP4 with I = 512 from half a row to 64 rows per expert: both GEMMs
    // on the persistent weight streams, blocks of 16, 32 or 64 rows by the
    // expected rows per expert (the tuner's choice for the TP2 shard)
    if (persist && md == 1 && I == 4 * 128 && rows >= 0.5 && rows < 64.0) {
        const int want = rows < 16.0 ? 16 : (rows < 32.0 ? 32 : 64);
        for (c = 0; c < kNumConfigs; ++c)
            if (kConfigs[c].bm == want && kConfigs[c].persist == 4 && kConfigs[c].persist2 == 1 &&
                persist_fits(kConfigs[c], md, bucket * k, E_local, H, I))
                return c;
    }
    // MXFP4 with I = 512: gemm2 on the multi-tile weight stream (one align)
    // from 2 tokens up to about 32 rows per expert
    if (md == 1 && I == 4 * 128 && rows > 0.025 && rows < 32.0) {
        const int want_bm = rows >= 8.0 ? 32 : 16, want_wk = rows < 0.5 ? 2 : 1;
        const int want_nt = rows < 0.5 ? 2 : (rows < 2.0 ? 8 : 4);
        for (c = 0; c < kNumConfigs; ++c)
            if (kConfigs[c].bm == want_bm && kConfigs[c].wk1 == want_wk && kConfigs[c].wk2 == 1 &&
                kConfigs[c].nt2 == want_nt && !kConfigs[c].tile && kConfigs[c].g2 < 0)
                return c;
    }
    int bm;
    if (md == 1)    // the fp4 stream prefers short blocks; 128 rows spill
        bm = busy <= 32.0 ? 16 : 64;
    else
        bm = busy <= 16.0 ? 16 : (busy <= 32.0 ? 32 : (rows < 192.0 ? 64 : 128));
    const int64_t blocks = experts * std::max<int64_t>(1, (int64_t)(rows / bm + 0.999));
    int wk = 1;
    const int wk_max = md == 0 ? 2 : 4;   // bf16: a 4-way K split measured slower than 2
    while (wk < wk_max && (bm < 64 || wk < 2) && blocks * (I / (32 * (4 / wk))) < 1024) wk <<= 1;
    // gemm2 from an LDS-staged tile once enough experts are touched to fill
    // the chip with its wider workgroups and the gain covers the second align
    int g2 = -1;
    if (md == 0 && bm == 16 && rows >= 0.5 && tile_config(0, 4, H, I) >= 0) g2 = tile_config(0, 4, H, I);
    if (md == 1 && bm == 16 && rows >= 4.0 && tile_config(1, 3, H, I) >= 0) g2 = tile_config(1, 3, H, I);
    if (md == 1 && bm == 64 && tile_config(1, 2, H, I) >= 0) g2 = tile_config(1, 2, H, I);
    for (c = 0; c < kNumConfigs; ++c)
        if (kConfigs[c].bm == bm && kConfigs[c].wk1 == wk && kConfigs[c].nb == 4 && !kConfigs[c].tile &&
            kConfigs[c].g2 == g2)
            return c;
    for (c = 0; c < kNumConfigs; ++c)
        if (kConfigs[c].bm == bm && kConfigs[c].wk1 == wk && kConfigs[c].nb == 4 && !kConfigs[c].tile &&
            kConfigs[c].g2 < 0)
            return c;
    return 0;
}

// The tuned table's entry for this exact layer and bucket, else the rules.
int default_config(int mode, int64_t T, int64_t H, int64_t I, int64_t E, int64_t E_local, int64_t k) {
    const int bucket = bucket_of(T);
    for (const TunedRow& r : kTuned)
        if (r.mode == mode && r.H == H && r.I == I && r.E == E && r.E_local == E_local && r.k == k &&
            r.bucket == bucket && r.config >= 0 && r.config < kNumConfigs)
            return r.config;
    return heuristic_config(mode, T, H, I, E, E_local, k);
}

// One GEMM's resolved kernel: rows per sorted block, K split and column
// blocks per wave (register stream), or an LDS tile shape.
struct KSpec {
    int bm, wk, nb;
    int tile;         // 0: register weight stream; 1 + shape: LDS-tiled
    int nt = 1;       // register stream: column tiles per workgroup
    int persist = 0;  // MXFP4 gemm1: the persistent weight stream with this many waves
};

struct Plan {
    int mode;
    int64_t T, H, I, E, k, A;
    KSpec ks[2];           // gemm1, gemm2
    int cfg_index;
    int64_t cap[2];        // sorted capacity of each GEMM's block size
    bool two_aligns;       // the GEMMs use different block sizes
    bool pack_x;
    int64_t e_off;         // global id of local expert 0
    bool y_out;            // per-slot rows go to the caller's y_rows; no combine
    int64_t y_row;         // element stride between the rows of y
    bool norm;             // RMSNorm pre-pass into the xn segment
    bool fuse;             // gemm2 and the combine in one kernel (no y, no second layout)
    bool small1;           // gemm1 per slot, without the align (implies fuse)
    bool norm_fold;        // the per-slot gemm1 normalises its token rows itself (no RMSNorm launch)
    bool norm_via_pack;    // a strided x is re-laid out (in the align launch), then normalised by rows
    // workspace offsets
    size_t off_counts, off_sorted[2], off_bexp[2], off_npad[2], off_eblk[2], off_x, off_xs, off_xn, off_xp, off_h, off_hs, off_y,
        total;
};

int kstep(int mode) { return mode == MOE_MODE_MXFP4 ? 128 : 32; }

// Element stride between consecutive flat rows a = t*k + j of a [T, k, H]
// y_rows tensor whose token stride is k times its slot stride.
int64_t y_rows_stride(const moe_tensor_t& y) {
    const int64_t T = y.size[0], k = y.size[1], H = y.size[2];
    if (k > 1) return y.stride[1];
    return T > 1 ? y.stride[0] : H;
}

// RMSNorm weight: [H] bf16 or fp32, any stride.
int check_norm_weight(const moe_tensor_t* w, int64_t H) {
    if (!w) return fail(MOE_ERR_NULL, "norm weight descriptor is NULL");
    int rc;
    if (w->dtype != MOE_DT_BF16 && w->dtype != MOE_DT_F32)
        return fail(MOE_ERR_DTYPE, "norm weight: dtype %s, expected bf16 or f32", dtype_name(w->dtype));
    if ((rc = check_desc(w, "norm weight", w->dtype, 1))) return rc;
    if (w->size[0] != H)
        return fail(MOE_ERR_SHAPE, "norm weight: size %lld, expected H = %lld", (long long)w->size[0], (long long)H);
    return MOE_OK;
}

void norm_params(NormParams* np, const moe_tensor_t& x, const moe_tensor_t& w, float eps) {
    np->x = (const uint16_t*)x.data;
    np->xs_t = x.stride[0];
    np->xs_h = x.size[1] > 1 ? x.stride[1] : 1;
    np->w = w.data;
    np->w_f32 = w.dtype == MOE_DT_F32 ? 1 : 0;
    np->ws = w.size[0] > 1 ? w.stride[0] : 1;
    np->eps = eps;
    np->T = x.size[0];
    np->H = x.size[1];
}

// Validate a fused call and build its plan. No device calls.
int plan_fused(const moe_fused_args_t* a, Plan* pl) {
    if (!a) return fail(MOE_ERR_NULL, "args is NULL");
    if (a->mode != MOE_MODE_BF16 && a->mode != MOE_MODE_MXFP4)
        return fail(MOE_ERR_ARG, "mode %d is not MOE_MODE_BF16 or MOE_MODE_MXFP4", a->mode);
    if (a->activation != MOE_ACT_SILU) return fail(MOE_ERR_ARG, "activation %d unsupported", a->activation);
    const bool fp4 = a->mode == MOE_MODE_MXFP4;
    int rc;
    if ((rc = check_desc(&a->x, "x", MOE_DT_BF16, 2))) return rc;
    const int64_t T = a->x.size[0], H = a->x.size[1];
    const int wdt = fp4 ? MOE_DT_FP4X2 : MOE_DT_BF16;
    if ((rc = check_desc(&a->gate, "gate", wdt, 3))) return rc;
    if ((rc = check_desc(&a->up, "up", wdt, 3))) return rc;
    if ((rc = check_desc(&a->w2, "w2", wdt, 3))) return rc;
    const int64_t E = a->gate.size[0], I = a->gate.size[1];
    const int64_t Hw = fp4 ? H / 2 : H, Iw = fp4 ? I / 2 : I;
    if (fp4 && (H % 2 != 0)) return fail(MOE_ERR_SHAPE, "x: H = %lld must be even in MXFP4 mode", (long long)H);
    if (a->gate.size[2] != Hw)
        return fail(MOE_ERR_SHAPE, "gate: hidden size %lld does not match x (H = %lld)", (long long)a->gate.size[2],
                    (long long)H);
    if ((rc = check_shape(a->up, "up", {E, I, Hw}))) return rc;
    if ((rc = check_shape(a->w2, "w2", {E, H, Iw}))) return rc;
    if (fp4) {
        if ((rc = check_desc(&a->gate_scale, "gate_scale", MOE_DT_E8M0, 3))) return rc;
        if ((rc = check_desc(&a->up_scale, "up_scale", MOE_DT_E8M0, 3))) return rc;
        if ((rc = check_desc(&a->w2_scale, "w2_scale", MOE_DT_E8M0, 3))) return rc;
        if ((rc = check_shape(a->gate_scale, "gate_scale", {E, I, H / 32}))) return rc;
        if ((rc = check_shape(a->up_scale, "up_scale", {E, I, H / 32}))) return rc;
        if ((rc = check_shape(a->w2_scale, "w2_scale", {E, H, I / 32}))) return rc;
    }
    if ((rc = check_desc(&a->topk_ids, "topk_ids", MOE_DT_I32, 2))) return rc;
    if ((rc = check_desc(&a->topk_weights, "topk_weights", MOE_DT_F32, 2))) return rc;
    const int64_t k = a->topk_ids.size[1];
    if ((rc = check_shape(a->topk_ids, "topk_ids", {T, k}))) return rc;
    if ((rc = check_shape(a->topk_weights, "topk_weights", {T, k}))) return rc;
    // expert-parallel shard: global ids, local experts [e_off, e_off + E)
    if (a->expert_offset < 0) return fail(MOE_ERR_ARG, "expert_offset = %d is negative", a->expert_offset);
    if (a->num_global_experts < 0 ||
        (a->num_global_experts > 0 && (int64_t)a->num_global_experts < (int64_t)a->expert_offset + E))
        return fail(MOE_ERR_ARG, "num_global_experts = %d below expert_offset + E = %lld", a->num_global_experts,
                    (long long)a->expert_offset + E);
    const int64_t E_cfg = a->num_global_experts > 0 ? a->num_global_experts : E;
    const bool norm = a->norm_weight.data != nullptr;
    if (norm) {
        if ((rc = check_norm_weight(&a->norm_weight, H))) return rc;
        if (!(a->norm_eps >= 0.f) || a->norm_eps == __builtin_inff())
            return fail(MOE_ERR_ARG, "norm_eps must be finite and >= 0");
    }
    const bool y_out = a->y_rows.data != nullptr;
    if (y_out) {
        if ((rc = check_desc(&a->y_rows, "y_rows", MOE_DT_BF16, 3))) return rc;
        if ((rc = check_shape(a->y_rows, "y_rows", {T, k, H}))) return rc;
        const moe_tensor_t& y = a->y_rows;
        const int64_t row = y_rows_stride(y);
        if ((H > 1 && y.stride[2] != 1) || row < H || (k > 1 && T > 1 && y.stride[0] != k * y.stride[1]) ||
            !aligned16(y.data) || (row * 2) % 16 != 0)
            return fail(MOE_ERR_LAYOUT,
                        "y_rows: needs last stride 1, stride(0) == k * stride(1) and 16-byte aligned rows");
    } else {
        if ((rc = check_desc(&a->out, "out", MOE_DT_BF16, 2))) return rc;
        if ((rc = check_shape(a->out, "out", {T, H}))) return rc;
    }

    // sizes the library handles
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %lld outside [1, 1024]", (long long)E);
    if (E_cfg > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED, "num_global_experts = %lld too large", (long long)E_cfg);
    if (k < 1 || k > 64) return fail(MOE_ERR_UNSUPPORTED, "k = %lld outside [1, 64]", (long long)k);
    const int ks = kstep(a->mode);
    if (H < ks || I < ks || H % 64 != 0 || H % ks != 0 || I % ks != 0 || I % 32 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "H = %lld and I = %lld must be multiples of %d (and H of 64)",
                    (long long)H, (long long)I, std::max(ks, 32));
    if (T > (int64_t)1 << 24 || T * k > ((int64_t)1 << 30))
        return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld too large", (long long)(T * k));

    // weight layouts: last dim contiguous, 16-byte aligned rows and experts
    const moe_tensor_t* ws[3] = {&a->gate, &a->up, &a->w2};
    const char* wn[3] = {"gate", "up", "w2"};
    const int eb = elem_bytes(wdt);
    for (int i = 0; i < 3; ++i) {
        const moe_tensor_t& w = *ws[i];
        if (w.stride[2] != 1) return fail(MOE_ERR_LAYOUT, "%s: last-dim stride must be 1", wn[i]);
        if (!aligned16(w.data) || ((w.stride[1] * eb) % 16) != 0 || ((w.stride[0] * eb) % 16) != 0)
            return fail(MOE_ERR_LAYOUT, "%s: rows and experts must start on 16-byte boundaries", wn[i]);
    }
    if (fp4) {
        // each lane reads a window of 4 * ring-steps scale bytes per row at once
        const moe_tensor_t* ss[3] = {&a->gate_scale, &a->up_scale, &a->w2_scale};
        const char* sn[3] = {"gate_scale", "up_scale", "w2_scale"};
        for (int i = 0; i < 3; ++i) {
            const moe_tensor_t& t = *ss[i];
            const int64_t K = t.size[2] * 32;
            const int64_t al = (K % 512 == 0) ? 16 : 8;
            if (t.stride[2] != 1) return fail(MOE_ERR_LAYOUT, "%s: last-dim stride must be 1", sn[i]);
            if (((uintptr_t)t.data % al) != 0 || (t.stride[1] % al) != 0 || (t.stride[0] % al) != 0)
                return fail(MOE_ERR_LAYOUT, "%s: rows and experts must start on %lld-byte boundaries", sn[i],
                            (long long)al);
        }
    }
    // outputs must not alias inputs
    const moe_tensor_t* ins[7] = {&a->x, &a->gate, &a->up, &a->w2, &a->topk_ids, &a->topk_weights, &a->norm_weight};
    const moe_tensor_t& dst = y_out ? a->y_rows : a->out;
    for (auto* t : ins)
        if (overlaps(dst, *t)) return fail(MOE_ERR_LAYOUT, "%s overlaps an input", y_out ? "y_rows" : "out");

    // configuration
    int ci = a->force_config;
    if (ci < 0) {
        ci = default_config(a->mode, T, H, I, E_cfg, E, k);
        // a tuned gemm2 fused with the combine cannot write per-slot rows
        if (y_out && ci < kNumConfigs && kConfigs[ci].fuse) ci = heuristic_config(a->mode, T, H, I, E_cfg, E, k);
        // a persistent stream that cannot run here (too many items for this
        // device's compute units): the per-item streams instead
        if (ci < kNumConfigs && !persist_fits(kConfigs[ci], fp4 ? 1 : 0, T * k, E, H, I))
            ci = heuristic_config(a->mode, T, H, I, E_cfg, E, k, false);
    }
    if (ci >= kNumConfigs) return fail(MOE_ERR_ARG, "force_config %d out of range", ci);
    const Cfg c1 = kConfigs[ci];
    Cfg c2 = c1.g2 >= 0 ? kConfigs[c1.g2] : c1;
    const int md = fp4 ? 1 : 0;
    // resolve and check one GEMM's kernel; the split of K is a preference:
    // halve it until every wave's share of K is a whole number of pipelined
    // chunks
    auto resolve = [&](const Cfg& c, int stage, KSpec* ks) -> int {
        const int64_t K = stage == 1 ? H : I, N = stage == 1 ? I : H;
        *ks = KSpec{c.bm, stage == 1 ? c.wk1 : c.wk2, c.nb, c.tile, stage == 2 ? c.nt2 : 1};
        if (c.tile) {
            const int shape = c.tile - 1;
            if (!gemm_tile_supported(md, shape))
                return fail(MOE_ERR_UNSUPPORTED, "config %d: tile shape not built for this mode", ci);
            ks->bm = gemm_tile_rows(md, shape);
            const int gran = gemm_tile_k_granule(md, shape);
            if (K % gran != 0 || N % gemm_tile_cols(shape, stage) != 0)
                return fail(MOE_ERR_UNSUPPORTED, "config %d: gemm%d needs K %% %d == 0 and N %% %d == 0", ci, stage,
                            gran, gemm_tile_cols(shape, stage));
            if ((shape == 6 || shape == 7) && (stage != 2 || !gemm2_rows_supported(K, N, T * k, y_out ? y_rows_stride(a->y_rows) : H)))
                return fail(MOE_ERR_UNSUPPORTED,
                            "config %d: the register-resident gemm2 needs K = 512 and y rows below 4 GB", ci);
            return MOE_OK;
        }
        if (stage == 2 && c.persist2) {
            if (md != 1 || !gemm2_persist_supported(c.bm, K, N) ||
                align_capacity(T * k, E, c.bm) / c.bm * (N / 256) > (int64_t)device_cus() * 256)
                return fail(MOE_ERR_UNSUPPORTED,
                            "config %d: the persistent gemm2 needs MXFP4, K = 512, N %% 256 == 0 and at most 256 "
                            "items per compute unit", ci);
            ks->wk = 1;
            ks->persist = 1;
            return MOE_OK;
        }
        if (stage == 1 && c.persist) {
            // one workgroup per compute unit, at most 256 items each
            if (md != 1 || !gemm1_persist_supported(c.bm, c.persist, K, N) ||
                align_capacity(T * k, E, c.bm) / c.bm * (N / (32 * c.persist)) > (int64_t)device_cus() * 256)
                return fail(MOE_ERR_UNSUPPORTED,
                            "config %d: the persistent gemm1 needs MXFP4, K in {2048, 4096, 8192}, N %% %d == 0 "
                            "and at most 256 items per compute unit", ci, 32 * c.persist);
            ks->wk = 1;
            ks->persist = c.persist;
            return MOE_OK;
        }
        int w = ks->wk;
        while (w > 1 && K % ((int64_t)gemm_k_granule(GemmKernelId{md, stage, c.bm, w, 0, c.nb}) * w) != 0) w >>= 1;
        ks->wk = w;
        const int gran = gemm_k_granule(GemmKernelId{md, stage, c.bm, 1, 0, c.nb});
        if (K % gran != 0)
            return fail(MOE_ERR_UNSUPPORTED, "config %d: gemm%d K = %lld must be a multiple of %d", ci, stage,
                        (long long)K, gran);
        GemmKernelId id{md, stage, c.bm, w, gemm_ring_steps(a->mode, c.bm, c.nb, w, K / w), c.nb, ks->nt};
        if (ks->nt != 1 && K != 4 * 128)
            return fail(MOE_ERR_UNSUPPORTED, "config %d: multi-tile gemm2 needs K = 512", ci);
        if (!gemm_supported(id)) return fail(MOE_ERR_UNSUPPORTED, "config %d not built", ci);
        if (N % gemm_tile_n(id) != 0)
            return fail(MOE_ERR_UNSUPPORTED, "config %d: gemm%d N not a multiple of the tile width", ci, stage);
        return MOE_OK;
    };
    if ((rc = resolve(c1, 1, &pl->ks[0]))) return rc;
    pl->fuse = c1.fuse != 0;
    pl->small1 = c1.fuse == 2;
    if (pl->fuse) {
        if (fp4 ? I != 4 * 128 : !gemm2_combine_bf16_supported(I))
            return fail(MOE_ERR_UNSUPPORTED,
                        "config %d: fused gemm2 + combine needs I = 512 (MXFP4) or I in {512, 768, ..., 1536} (bf16)",
                        ci);
        // one workgroup of up to 1024 threads per (token, 16 columns); a
        // launch holds fewer than 2^32 threads
        if (H % 16 != 0 || T * (H / 16) * 1024 >= ((int64_t)1 << 32))
            return fail(MOE_ERR_UNSUPPORTED,
                        "config %d: fused gemm2 + combine needs H %% 16 == 0 and T * H / 16 < 2^22", ci);
        if (pl->small1 && (H % 2048 != 0 || H > 8192 || T * k > (1 << 16)))
            return fail(MOE_ERR_UNSUPPORTED,
                        "config %d: gemm1 per slot needs H %% 2048 == 0, H <= 8192 and T*k <= 65536", ci);
        if (y_out) return fail(MOE_ERR_UNSUPPORTED, "config %d: fused gemm2 + combine writes out, not y_rows", ci);
        pl->ks[1] = pl->ks[0];   // no second layout
    } else if ((rc = resolve(c2, 2, &pl->ks[1]))) {
        // a chosen (not forced) register-resident gemm2 whose y rows would
        // span 4 GB or more: the LDS tile with the same block rows instead
        if (a->force_config >= 0 || !(c2.tile == 7 || c2.tile == 8)) return rc;
        c2 = kConfigs[c2.bm == 256 ? 11 : 38];
        if ((rc = resolve(c2, 2, &pl->ks[1]))) return rc;
    }

    pl->mode = a->mode;
    pl->T = T;
    pl->H = H;
    pl->I = I;
    pl->E = E;
    pl->k = k;
    pl->A = T * k;
    pl->cfg_index = ci;
    pl->e_off = a->expert_offset;
    pl->y_out = y_out;
    pl->y_row = y_out ? y_rows_stride(a->y_rows) : H;
    pl->cap[0] = align_capacity(pl->A, E, pl->ks[0].bm);
    pl->cap[1] = align_capacity(pl->A, E, pl->ks[1].bm);
    pl->two_aligns = pl->ks[0].bm != pl->ks[1].bm;
    const bool x_direct = a->x.stride[1] == 1 && aligned16(a->x.data) &&
                          (T <= 1 || (a->x.stride[0] * 2) % 16 == 0);
    pl->norm = norm;
    // Each per-slot gemm1 workgroup normalising its own token row saves the
    // RMSNorm launch (measured: 8-9 us of norm cost down to 3-5 us at T = 1
    // and 4) but repeats the row's reduction once per workgroup, which loses
    // from about 16 tokens (MXFP4 T = 16: 15 against 8 us). Same bits either way.
    pl->norm_fold = norm && pl->small1 && T <= 8;
    // bf16 rows with a non-unit last-dim stride are laid out into the
    // workspace for the GEMMs that stage whole 16-byte row chunks (one pass,
    // coalesced along the stride-1 dimension); gemm1 per slot reads x
    // through both strides itself
    pl->pack_x = !fp4 && !x_direct && !norm && !pl->small1;
    // With the RMSNorm on the aligned path, x with a non-unit last-dim
    // stride is re-laid out by the align launch's spare workgroups and then
    // normalised by rows (a launch of its own: it needs the whole row); the
    // column-layout norm would leave few workgroups each reading 64 rows
    pl->norm_via_pack = norm && !pl->norm_fold && !pl->small1 && H > 1 && a->x.stride[1] != 1;
    {
        // the tiled kernels address every operand row with a 32-bit offset
        const int64_t eb = fp4 ? 1 : 2;
        const int64_t x_row = fp4 ? H / 2 : (pl->pack_x || norm ? H * 2 : a->x.stride[0] * 2);
        const int64_t lim = (int64_t)1 << 31;
        if (pl->ks[0].tile && (T * x_row >= lim || I * a->gate.stride[1] * eb >= lim ||
                               I * a->up.stride[1] * eb >= lim))
            return fail(MOE_ERR_UNSUPPORTED, "config %d: operands too large for the tiled gemm1", ci);
        if (pl->ks[1].tile && (pl->A * I * eb >= lim || H * a->w2.stride[1] * eb >= lim))
            return fail(MOE_ERR_UNSUPPORTED, "config %d: operands too large for the tiled gemm2", ci);
    }

    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    pl->off_counts = take(align_scratch_bytes(pl->A, (int32_t)E));
    for (int g = 0; g < 2; ++g) {
        if (g == 1 && !pl->two_aligns) {
            pl->off_sorted[1] = pl->off_sorted[0];
            pl->off_bexp[1] = pl->off_bexp[0];
            pl->off_npad[1] = pl->off_npad[0];
            pl->off_eblk[1] = pl->off_eblk[0];
            break;
        }
        pl->off_sorted[g] = take((size_t)pl->cap[g] * 4);
        pl->off_bexp[g] = take((size_t)(pl->cap[g] / pl->ks[g].bm) * 4);
        pl->off_npad[g] = take(4);
        pl->off_eblk[g] = take((size_t)(E + 1) * 4);
    }
    pl->off_x = pl->off_xs = pl->off_xn = pl->off_xp = 0;
    // normalised rows, bf16 (unless the per-slot gemm1 normalises in LDS)
    if (norm && !pl->norm_fold) pl->off_xn = take((size_t)T * (size_t)H * 2);
    if (pl->norm_via_pack) pl->off_xp = take((size_t)T * (size_t)H * 2);
    if (fp4) {
        pl->off_x = take((size_t)T * (size_t)(H / 2));
        pl->off_xs = take((size_t)T * (size_t)(H / 32));
    } else if (pl->pack_x) {
        pl->off_x = take((size_t)T * (size_t)H * 2);
    }
    // h rows by flat assignment index
    if (fp4) {
        pl->off_h = take((size_t)pl->A * (size_t)(I / 2));
        pl->off_hs = take((size_t)pl->A * (size_t)(I / 32));
    } else {
        pl->off_h = take((size_t)pl->A * (size_t)I * 2);
        pl->off_hs = 0;
    }
    pl->off_y = (y_out || pl->fuse) ? 0 : take((size_t)pl->A * (size_t)H * 2);   // y: bf16 (or y_rows; none fused)
    pl->total = off;
    return MOE_OK;
}

// ------------------------------------------------------------ backward

struct BwdPlan {
    Plan fwd;              // the forward's checked sizes
    int64_t cap;           // sorted capacity at block_m 64
    bool pack_x, pack_d;   // activation rows re-laid out (unit stride, aligned)
    bool wgrad_f32;
    size_t off_counts, off_sorted, off_bexp, off_npad, off_ebf, off_ebl, off_xp, off_dp, off_gu, off_q, off_dgu,
        off_wh, off_dxa, total;
};

constexpr int kBwdBM = 64;       // sorted block rows (one K stage of the weight-gradient GEMMs)
constexpr int kBwdWgradBM = 128; // weight-space rows per weight-gradient tile

// A weight gradient output: f32 or bf16, last stride 1, rows aligned for the
// epilogue's 4-element stores.
int check_wgrad(const moe_tensor_t* t, const char* name, std::initializer_list<int64_t> shape, int* dtype) {
    if (!t) return fail(MOE_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->dtype != MOE_DT_F32 && t->dtype != MOE_DT_BF16)
        return fail(MOE_ERR_DTYPE, "%s: dtype %s, expected f32 or bf16", name, dtype_name(t->dtype));
    int rc;
    if ((rc = check_desc(t, name, t->dtype, 3))) return rc;
    if ((rc = check_shape(*t, name, shape))) return rc;
    const int64_t al = t->dtype == MOE_DT_F32 ? 16 : 8, eb = elem_bytes(t->dtype);
    if (t->stride[2] != 1 || ((uintptr_t)t->data % al) != 0 || (t->stride[1] * eb) % al != 0 ||
        (t->stride[0] * eb) % al != 0)
        return fail(MOE_ERR_LAYOUT, "%s: needs last stride 1 and %lld-byte aligned rows", name, (long long)al);
    *dtype = t->dtype;
    return MOE_OK;
}

bool rows_direct(const moe_tensor_t& x) {
    return x.stride[1] == 1 && aligned16(x.data) && (x.size[0] <= 1 || (x.stride[0] * 2) % 16 == 0);
}

int plan_bwd(const moe_bwd_args_t* b, BwdPlan* pl) {
    if (!b) return fail(MOE_ERR_NULL, "args is NULL");
    if (b->fwd.mode != MOE_MODE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the backward is built for bf16 mode only");
    if (b->fwd.y_rows.data || b->fwd.norm_weight.data)
        return fail(MOE_ERR_UNSUPPORTED, "the backward takes neither y_rows nor norm_weight");
    moe_fused_args_t fa = b->fwd;
    fa.out = b->dx;          // dx takes out's place in the forward's checks
    fa.force_config = -1;
    int rc;
    if ((rc = plan_fused(&fa, &pl->fwd))) return rc;
    const Plan& f = pl->fwd;
    const int64_t T = f.T, H = f.H, I = f.I, E = f.E, k = f.k, A = f.A;
    if (H % 128 != 0 || I % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "backward: H = %lld and I = %lld must be multiples of 128", (long long)H,
                    (long long)I);
    if ((rc = check_desc(&b->dout, "dout", MOE_DT_BF16, 2))) return rc;
    if ((rc = check_shape(b->dout, "dout", {T, H}))) return rc;
    int dt_g, dt_u, dt_2;
    if ((rc = check_wgrad(&b->dgate, "dgate", {E, I, H}, &dt_g))) return rc;
    if ((rc = check_wgrad(&b->dup, "dup", {E, I, H}, &dt_u))) return rc;
    if ((rc = check_wgrad(&b->dw2, "dw2", {E, H, I}, &dt_2))) return rc;
    if (dt_g != dt_u || dt_g != dt_2) return fail(MOE_ERR_DTYPE, "dgate, dup and dw2 must share one dtype");
    if ((rc = check_desc(&b->dtopk_weights, "dtopk_weights", MOE_DT_F32, 2))) return rc;
    if (b->accumulate != 0 && b->accumulate != 1) return fail(MOE_ERR_ARG, "accumulate must be 0 or 1");
    if ((rc = check_shape(b->dtopk_weights, "dtopk_weights", {T, k}))) return rc;
    const moe_tensor_t* ins[7] = {&b->fwd.x, &b->fwd.gate, &b->fwd.up, &b->fwd.w2, &b->fwd.topk_ids,
                                  &b->fwd.topk_weights, &b->dout};
    const moe_tensor_t* outs[5] = {&b->dx, &b->dgate, &b->dup, &b->dw2, &b->dtopk_weights};
    for (int i = 0; i < 5; ++i) {
        for (auto* t : ins)
            if (overlaps(*outs[i], *t)) return fail(MOE_ERR_LAYOUT, "a gradient output overlaps an input");
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(*outs[i], *outs[j]) && !interleaved_disjoint(*outs[i], *outs[j]))
                return fail(MOE_ERR_LAYOUT, "gradient outputs overlap each other");
    }
    pl->wgrad_f32 = dt_g == MOE_DT_F32;
    pl->pack_x = !rows_direct(b->fwd.x);
    pl->pack_d = !rows_direct(b->dout);
    pl->cap = align_capacity(A, (int32_t)E, kBwdBM);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    pl->off_counts = take(align_scratch_bytes(A, (int32_t)E));
    pl->off_sorted = take((size_t)pl->cap * 4);
    pl->off_bexp = take((size_t)(pl->cap / kBwdBM) * 4);
    pl->off_npad = take(4);
    pl->off_ebf = take((size_t)E * 4);
    pl->off_ebl = take((size_t)E * 4);
    pl->off_xp = pl->pack_x ? take((size_t)T * H * 2) : 0;
    pl->off_dp = pl->pack_d ? take((size_t)T * H * 2) : 0;
    pl->off_gu = take((size_t)A * 2 * I * 4);
    pl->off_q = take((size_t)A * I * 4);
    pl->off_dgu = take((size_t)A * 2 * I * 2);
    pl->off_wh = take((size_t)A * I * 2);
    pl->off_dxa = take((size_t)A * H * 4);
    pl->total = off;
    return MOE_OK;
}

struct StageTimer {
    void* const* ev;
    hipStream_t s;
    void begin(int st) const {
        if (ev && ev[2 * st]) (void)hipEventRecord((hipEvent_t)ev[2 * st], s);
    }
    void end(int st) const {
        if (ev && ev[2 * st + 1]) (void)hipEventRecord((hipEvent_t)ev[2 * st + 1], s);
    }
};

// Calls whose tokens exceed what one launch sequence can address (tiled
// operand offsets of 2^31 bytes, thread counts, T*k) run in chunks of this
// many tokens. Tokens are independent and every chunk takes the whole
// call's configuration (the bucket of the first chunk is the whole call's:
// buckets stop at 32768), so the result is what one launch would give.
constexpr int64_t kChunkT = 32768;

// The call restricted to tokens [t0, t0 + n): the per-token tensors' views
// (x, ids, weights, and out or y_rows) start at row t0 and hold n rows.
moe_fused_args_t token_slice(const moe_fused_args_t& a, int64_t t0, int64_t n) {
    moe_fused_args_t c = a;
    auto cut = [&](moe_tensor_t& t, int eb) {
        if (t.data) t.data = (char*)t.data + t0 * t.stride[0] * eb;
        t.size[0] = n;
    };
    cut(c.x, 2);
    cut(c.topk_ids, 4);
    cut(c.topk_weights, 4);
    if (c.y_rows.data)
        cut(c.y_rows, 2);
    else
        cut(c.out, 2);
    return c;
}

// plan_fused, or, when the whole call is too large for one launch sequence
// and the configuration is the built-in choice, the plan of one chunk of
// kChunkT tokens (*chunk = kChunkT; 0 when the call runs whole).
int plan_auto(const moe_fused_args_t* a, Plan* pl, int64_t* chunk) {
    *chunk = 0;
    const int rc = plan_fused(a, pl);
    if (rc != MOE_ERR_UNSUPPORTED || a->force_config >= 0 || a->x.size[0] <= kChunkT) return rc;
    const std::string why = g_last_error;
    const moe_fused_args_t c = token_slice(*a, 0, kChunkT);
    if (plan_fused(&c, pl) != MOE_OK) {
        g_last_error = why;
        return rc;
    }
    *chunk = kChunkT;
    return MOE_OK;
}

// The launches of one planned fused call: align, (prepare), gemm1 + act,
// gemm2, combine. The plan has been checked; base is the workspace.
int run_fused(const moe_fused_args_t& a, const Plan& pl, char* base, hipStream_t s) {
    const StageTimer tm{a.stage_events, s};
    const bool fp4 = pl.mode == MOE_MODE_MXFP4;
    int32_t *sorted[2], *bexp[2], *npad[2], *eblk[2];
    for (int g = 0; g < 2; ++g) {
        sorted[g] = (int32_t*)(base + pl.off_sorted[g]);
        bexp[g] = (int32_t*)(base + pl.off_bexp[g]);
        npad[g] = (int32_t*)(base + pl.off_npad[g]);
        eblk[g] = (int32_t*)(base + pl.off_eblk[g]);
    }
    hipError_t e;

    // The activation operand of gemm1 is prepared by the spare workgroups of
    // the align launch (its first launch when the align takes three): the
    // RMSNorm (then, in MXFP4 mode, the quantisation of the normalised rows),
    // the MXFP4 quantisation, or the bf16 re-layout of a strided x. The
    // per-slot gemm1 (no align) reads x itself, folding the norm in.
    PrepParams pr{};
    int prep = 0;
    const void* a_op = a.x.data;
    int64_t a_row = a.x.stride[0];
    if (fp4) {
        pr.q.src = (const uint16_t*)a.x.data;
        pr.q.E = 1;
        pr.q.R = pl.T;
        pr.q.K = pl.H;
        pr.q.ss_r = a.x.stride[0];
        pr.q.ss_k = a.x.stride[1];
        pr.q.codes = (uint8_t*)(base + pl.off_x);
        pr.q.cs_r = pl.H / 2;
        pr.q.scales = (uint8_t*)(base + pl.off_xs);
        pr.q.xs_r = pl.H / 32;
    }
    if (!pl.small1) {
        if (pl.norm) {
            norm_params(&pr.n, a.x, a.norm_weight, a.norm_eps);
            pr.n.out = (uint16_t*)(base + pl.off_xn);
            pr.n.os_t = pl.H;
            pr.n.os_h = 1;
            prep = kPrepNormRows;
            if (pl.norm_via_pack) {
                // the align launch re-lays x out; the norm follows in stage 1
                prep = kPrepPack;
                pr.pk.src = (const uint16_t*)a.x.data;
                pr.pk.s_t = a.x.stride[0];
                pr.pk.s_h = a.x.stride[1];
                pr.pk.dst = (uint16_t*)(base + pl.off_xp);
                pr.pk.T = pl.T;
                pr.pk.H = pl.H;
                pr.n.x = pr.pk.dst;
                pr.n.xs_t = pl.H;
                pr.n.xs_h = 1;
            }
            a_op = base + pl.off_xn;
            a_row = pl.H;
            if (fp4) {
                pr.quant_after = 1;
                pr.q.src = (const uint16_t*)(base + pl.off_xn);
                pr.q.ss_r = pl.H;
                pr.q.ss_k = 1;
            }
        } else if (fp4) {
            prep = kPrepQuant;
        } else if (pl.pack_x) {
            prep = kPrepPack;
            pr.pk.src = (const uint16_t*)a.x.data;
            pr.pk.s_t = a.x.stride[0];
            pr.pk.s_h = a.x.stride[1];
            pr.pk.dst = (uint16_t*)(base + pl.off_x);
            pr.pk.T = pl.T;
            pr.pk.H = pl.H;
            a_op = base + pl.off_x;
            a_row = pl.H;
        }
        if (fp4) {
            a_op = base + pl.off_x;
            a_row = pl.H / 2;
        }
    }

    // stage 0: align (with the preparation); when the two GEMMs use
    // different block sizes, the same pass writes the second padded layout
    tm.begin(0);
    if (!pl.small1) {
        AlignParams ap{};
        ap.ids = (const int32_t*)a.topk_ids.data;
        ap.is_t = a.topk_ids.stride[0];
        ap.is_j = a.topk_ids.stride[1];
        ap.T = (int32_t)pl.T;
        ap.k = (int32_t)pl.k;
        ap.A = (int32_t)pl.A;
        ap.E = (int32_t)pl.E;
        ap.e_off = pl.e_off;
        ap.bm = pl.ks[0].bm;
        ap.cap = (int32_t)pl.cap[0];
        ap.sorted = sorted[0];
        ap.block_expert = bexp[0];
        ap.n_padded = npad[0];
        ap.counts = (int32_t*)(base + pl.off_counts);
        ap.expert_block = eblk[0];
        if (pl.two_aligns) {
            ap.bm2 = pl.ks[1].bm;
            ap.cap2 = (int32_t)pl.cap[1];
            ap.sorted2 = sorted[1];
            ap.block_expert2 = bexp[1];
            ap.n_padded2 = npad[1];
            ap.expert_block2 = eblk[1];
        }
        if ((e = launch_align_prep(ap, prep, pr, s)) != hipSuccess) return hip_fail(e, "align");
    }
    tm.end(0);
    // stage 1: the RMSNorm (and MXFP4 quantisation) of a re-laid-out x, and
    // the RMSNorm of a per-slot gemm1 call that does not fold it in (there is
    // no align launch), have launches of their own
    tm.begin(1);
    if (pl.norm_via_pack && (e = launch_prep_norm_rows(pr, s)) != hipSuccess) return hip_fail(e, "rmsnorm");
    if (pl.small1 && pl.norm && !pl.norm_fold) {
        NormParams np{};
        norm_params(&np, a.x, a.norm_weight, a.norm_eps);
        np.out = (uint16_t*)(base + pl.off_xn);
        np.os_t = pl.H;
        np.os_h = 1;
        if ((e = launch_rmsnorm(np, s)) != hipSuccess) return hip_fail(e, "rmsnorm");
    }
    tm.end(1);

    // launch one GEMM with its resolved kernel
    auto launch = [&](int g, const GemmParams& gp) -> hipError_t {
        const KSpec& k = pl.ks[g];
        if (k.tile) return launch_gemm_tile(fp4 ? 1 : 0, k.tile - 1, g + 1, gp, s);
        if (k.persist) return g == 0 ? launch_gemm1_persist(k.bm, k.persist, gp, s) : launch_gemm2_persist(k.bm, gp, s);
        GemmKernelId id{fp4 ? 1 : 0, g + 1, k.bm, k.wk,
                        gemm_ring_steps(pl.mode, k.bm, k.nb, k.wk, (g == 0 ? pl.H : pl.I) / k.wk), k.nb, k.nt};
        return launch_gemm(id, gp, s);
    };
    // stage 2: gemm1 + SiLU(gate) * up
    tm.begin(2);
    if (pl.small1) {
        // per slot, from the bf16 activation (or its normalised rows)
        Gemm1SmallParams sp{};
        sp.x = pl.norm && !pl.norm_fold ? (const uint16_t*)(base + pl.off_xn) : (const uint16_t*)a.x.data;
        sp.xs_t = pl.norm && !pl.norm_fold ? pl.H : a.x.stride[0];
        sp.xs_h = pl.norm && !pl.norm_fold ? 1 : (pl.H > 1 ? a.x.stride[1] : 1);
        if (pl.norm_fold) {
            // the RMSNorm is folded into this gemm1 (same order, same bits)
            NormParams np{};
            norm_params(&np, a.x, a.norm_weight, a.norm_eps);
            sp.nw = np.w;
            sp.nws = np.ws;
            sp.nw_f32 = np.w_f32;
            sp.eps = np.eps;
        }
        sp.gate = (const uint8_t*)a.gate.data;
        sp.up = (const uint8_t*)a.up.data;
        sp.g_e = a.gate.stride[0];
        sp.g_r = a.gate.stride[1];
        sp.u_e = a.up.stride[0];
        sp.u_r = a.up.stride[1];
        sp.gate_sc = (const uint8_t*)a.gate_scale.data;
        sp.up_sc = (const uint8_t*)a.up_scale.data;
        sp.gs_e = a.gate_scale.stride[0];
        sp.gs_r = a.gate_scale.stride[1];
        sp.us_e = a.up_scale.stride[0];
        sp.us_r = a.up_scale.stride[1];
        sp.ids = (const int32_t*)a.topk_ids.data;
        sp.is_t = a.topk_ids.stride[0];
        sp.is_j = a.topk_ids.stride[1];
        sp.e_off = pl.e_off;
        sp.E = (int32_t)pl.E;
        sp.k = (int32_t)pl.k;
        sp.A = (int32_t)pl.A;
        sp.H = (int32_t)pl.H;
        sp.I = (int32_t)pl.I;
        sp.hq = (uint8_t*)(base + pl.off_h);
        sp.hs = (uint8_t*)(base + pl.off_hs);
        if (!fp4) {
            // bf16 weights: byte strides
            sp.g_e *= 2;
            sp.g_r *= 2;
            sp.u_e *= 2;
            sp.u_r *= 2;
        }
        if ((e = fp4 ? launch_gemm1_small(sp, s) : launch_gemm1_small_bf16(sp, s)) != hipSuccess)
            return hip_fail(e, "gemm1");
    }
    GemmParams g1{};
    g1.sorted = sorted[0];
    g1.block_expert = bexp[0];
    g1.n_padded = npad[0];
    g1.A = (int32_t)pl.A;
    g1.k = (int32_t)pl.k;
    g1.E = (int32_t)pl.E;
    g1.a = a_op;
    g1.a_row = a_row;
    g1.a_sc = fp4 ? (const uint8_t*)(base + pl.off_xs) : nullptr;
    g1.a_sc_row = pl.H / 32;
    g1.b0 = a.gate.data;
    g1.b1 = a.up.data;
    g1.b0_e = a.gate.stride[0];
    g1.b0_r = a.gate.stride[1];
    g1.b1_e = a.up.stride[0];
    g1.b1_r = a.up.stride[1];
    if (fp4) {
        g1.b0_sc = (const uint8_t*)a.gate_scale.data;
        g1.b1_sc = (const uint8_t*)a.up_scale.data;
        g1.b0sc_e = a.gate_scale.stride[0];
        g1.b0sc_r = a.gate_scale.stride[1];
        g1.b1sc_e = a.up_scale.stride[0];
        g1.b1sc_r = a.up_scale.stride[1];
    }
    g1.K = (int32_t)pl.H;
    g1.N = (int32_t)pl.I;
    g1.out = base + pl.off_h;
    g1.out_sc = fp4 ? (uint8_t*)(base + pl.off_hs) : nullptr;
    g1.n_tile_groups = 2;
    g1.max_mblocks = (int32_t)(pl.cap[0] / pl.ks[0].bm);
    g1.expert_block = eblk[0];
    if (!pl.small1 && (e = launch(0, g1)) != hipSuccess) return hip_fail(e, "gemm1");
    tm.end(2);

    // the combine's arguments (the separate combine, or folded into gemm2)
    CombineParams cp{};
    cp.y = reinterpret_cast<const uint16_t*>(base + pl.off_y);
    cp.ys_t = pl.k * pl.H;
    cp.ys_j = pl.H;
    cp.e_off = pl.e_off;
    cp.ids = (const int32_t*)a.topk_ids.data;
    cp.is_t = a.topk_ids.stride[0];
    cp.is_j = a.topk_ids.stride[1];
    cp.w = (const float*)a.topk_weights.data;
    cp.ws_t = a.topk_weights.stride[0];
    cp.ws_j = a.topk_weights.stride[1];
    cp.out = (uint16_t*)a.out.data;
    cp.os_t = a.out.stride[0];
    cp.os_h = a.out.stride[1];
    cp.T = (int32_t)pl.T;
    cp.k = (int32_t)pl.k;
    cp.E = (int32_t)pl.E;
    cp.H = (int32_t)pl.H;

    // stage 3: gemm2
    tm.begin(3);
    GemmParams g2{};
    g2.sorted = sorted[1];
    g2.block_expert = bexp[1];
    g2.n_padded = npad[1];
    g2.A = (int32_t)pl.A;
    g2.k = (int32_t)pl.k;
    g2.E = (int32_t)pl.E;
    g2.a = base + pl.off_h;
    g2.a_row = fp4 ? pl.I / 2 : pl.I;
    g2.a_sc = fp4 ? (const uint8_t*)(base + pl.off_hs) : nullptr;
    g2.a_sc_row = pl.I / 32;
    g2.b0 = a.w2.data;
    g2.b0_e = a.w2.stride[0];
    g2.b0_r = a.w2.stride[1];
    if (fp4) {
        g2.b0_sc = (const uint8_t*)a.w2_scale.data;
        g2.b0sc_e = a.w2_scale.stride[0];
        g2.b0sc_r = a.w2_scale.stride[1];
    }
    g2.K = (int32_t)pl.I;
    g2.N = (int32_t)pl.H;
    g2.out = pl.y_out ? a.y_rows.data : (void*)(base + pl.off_y);
    g2.out_row = pl.y_row;
    g2.n_tile_groups = 2;
    g2.max_mblocks = (int32_t)(pl.cap[1] / pl.ks[1].bm);
    g2.expert_block = eblk[1];
    if (pl.fuse) {
        const Gemm2CombineParams gc{g2, cp};
        if ((e = fp4 ? launch_gemm2_combine(gc, s) : launch_gemm2_combine_bf16(gc, s)) != hipSuccess)
            return hip_fail(e, "gemm2");
    } else if ((e = launch(1, g2)) != hipSuccess) {
        return hip_fail(e, "gemm2");
    }
    tm.end(3);

    // stage 4: combine (the caller combines y_rows itself; fused into gemm2)
    tm.begin(4);
    if (!pl.y_out && !pl.fuse && (e = launch_combine(cp, s)) != hipSuccess) return hip_fail(e, "combine");
    tm.end(4);
    return ok();
}

}  // namespace

int moe::report_error(int status, const char* what, const char* detail) {
    return fail(status, "%s: %s", what, detail);
}

extern "C" {

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "tensor sizes do not match";
        case MOE_ERR_DTYPE: return "wrong element type";
        case MOE_ERR_LAYOUT: return "unsupported strides or alignment";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_UNSUPPORTED: return "sizes outside what the library supports";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_topk_softmax(const moe_tensor_t* logits, int32_t k, int32_t renorm, int32_t shared_id, float shared_w,
                     const moe_tensor_t* ids, const moe_tensor_t* weights, moe_stream_t stream) {
    int rc;
    if ((rc = check_desc(logits, "logits", MOE_DT_F32, 2))) return rc;
    const int64_t T = logits->size[0], E = logits->size[1];
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "logits: %lld experts outside [1, 1024]", (long long)E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_ERR_ARG, "k = %d outside [1, min(E, 32)]", k);
    if (renorm != 0 && renorm != 1) return fail(MOE_ERR_ARG, "renorm must be 0 or 1");
    const int64_t kt = k + (shared_id >= 0 ? 1 : 0);
    if ((rc = check_desc(ids, "ids", MOE_DT_I32, 2))) return rc;
    if ((rc = check_desc(weights, "weights", MOE_DT_F32, 2))) return rc;
    if ((rc = check_shape(*ids, "ids", {T, kt}))) return rc;
    if ((rc = check_shape(*weights, "weights", {T, kt}))) return rc;
    if (T > ((int64_t)1 << 31) - 4) return fail(MOE_ERR_UNSUPPORTED, "T too large");
    if (overlaps(*ids, *logits) || overlaps(*weights, *logits) || overlaps(*ids, *weights))
        return fail(MOE_ERR_LAYOUT, "outputs overlap inputs or each other");
    if (T == 0) return ok();
    RouteParams p{};
    p.logits = (const float*)logits->data;
    p.T = T;
    p.ls_t = logits->stride[0];
    p.ls_e = logits->stride[1];
    p.E = (int32_t)E;
    p.k = k;
    p.renorm = renorm;
    p.shared_id = shared_id;
    p.shared_w = shared_w;
    p.ids = (int32_t*)ids->data;
    p.is_t = ids->stride[0];
    p.is_j = ids->stride[1];
    p.w = (float*)weights->data;
    p.ws_t = weights->stride[0];
    p.ws_j = weights->stride[1];
    hipError_t e = launch_route(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "route");
    return ok();
}

int64_t moe_align_capacity(int64_t assignments, int32_t num_experts, int32_t block_m) {
    if (assignments < 0 || num_experts < 1 || !valid_bm(block_m)) return -1;
    return align_capacity(assignments, num_experts, block_m);
}

int moe_align_workspace_size(int64_t tokens, int32_t k, int32_t num_experts, int32_t block_m, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
    if (tokens < 0 || k < 1 || num_experts < 1 || num_experts > 1024 || !valid_bm(block_m))
        return fail(MOE_ERR_ARG, "invalid sizes");
    *bytes = round_up(align_scratch_bytes(tokens * k, num_experts), 256);
    return ok();
}

int moe_align(const moe_tensor_t* ids, int32_t num_experts, int32_t block_m, const moe_tensor_t* sorted_ids,
              const moe_tensor_t* block_expert, const moe_tensor_t* n_padded, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
    int rc;
    if ((rc = check_desc(ids, "ids", MOE_DT_I32, 2))) return rc;
    if (num_experts < 1 || num_experts > 1024)
        return fail(MOE_ERR_UNSUPPORTED, "num_experts = %d outside [1, 1024]", num_experts);
    if (!valid_bm(block_m)) return fail(MOE_ERR_ARG, "block_m = %d not in {16, 32, 64, 128, 256}", block_m);
    const int64_t T = ids->size[0], k = ids->size[1];
    if (k < 1) return fail(MOE_ERR_SHAPE, "ids: k must be >= 1");
    const int64_t A = T * k;
    if (A > ((int64_t)1 << 30)) return fail(MOE_ERR_UNSUPPORTED, "T*k too large");
    const int64_t cap = align_capacity(A, num_experts, block_m);
    if ((rc = check_desc(sorted_ids, "sorted_ids", MOE_DT_I32, 1))) return rc;
    if ((rc = check_desc(block_expert, "block_expert", MOE_DT_I32, 1))) return rc;
    if ((rc = check_desc(n_padded, "n_padded", MOE_DT_I32, 1))) return rc;
    if (sorted_ids->size[0] < cap || (sorted_ids->size[0] > 1 && sorted_ids->stride[0] != 1))
        return fail(MOE_ERR_SHAPE, "sorted_ids needs %lld contiguous entries", (long long)cap);
    if (block_expert->size[0] < cap / block_m || (block_expert->size[0] > 1 && block_expert->stride[0] != 1))
        return fail(MOE_ERR_SHAPE, "block_expert needs %lld contiguous entries", (long long)(cap / block_m));
    if (n_padded->size[0] < 1) return fail(MOE_ERR_SHAPE, "n_padded needs one entry");
    if (!n_padded->data) return fail(MOE_ERR_NULL, "n_padded: data is NULL");
    const size_t need = align_scratch_bytes(A, num_experts);
    if (need > 0 && (!ws || ((uintptr_t)ws & 255u) || ws_bytes < need))
        return fail(MOE_ERR_WORKSPACE, "align needs %zu bytes of 256-byte aligned scratch", need);
    if (overlaps(*sorted_ids, *ids) || overlaps(*block_expert, *ids) || overlaps(*n_padded, *ids))
        return fail(MOE_ERR_LAYOUT, "outputs overlap ids");
    AlignParams p{};
    p.ids = (const int32_t*)ids->data;
    p.is_t = ids->stride[0];
    p.is_j = ids->stride[1];
    p.T = (int32_t)T;
    p.k = (int32_t)k;
    p.A = (int32_t)A;
    p.E = num_experts;
    p.bm = block_m;
    p.cap = (int32_t)cap;
    p.sorted = (int32_t*)sorted_ids->data;
    p.block_expert = (int32_t*)block_expert->data;
    p.n_padded = (int32_t*)n_padded->data;
    p.counts = (int32_t*)ws;
    hipError_t e = launch_align(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "align");
    return ok();
}

int moe_quant_mxfp4(const moe_tensor_t* src, const moe_tensor_t* codes, const moe_tensor_t* scales,
                    moe_stream_t stream) {
    if (!src || !codes || !scales) return fail(MOE_ERR_NULL, "NULL descriptor");
    const int nd = src->ndim;
    if (nd != 2 && nd != 3) return fail(MOE_ERR_SHAPE, "src must have 2 or 3 dims");
    int rc;
    if ((rc = check_desc(src, "src", MOE_DT_BF16, nd))) return rc;
    if ((rc = check_desc(codes, "codes", MOE_DT_FP4X2, nd))) return rc;
    if ((rc = check_desc(scales, "scales", MOE_DT_E8M0, nd))) return rc;
    const int64_t K = src->size[nd - 1];
    if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED, "K = %lld must be a multiple of 32", (long long)K);
    for (int i = 0; i < nd - 1; ++i)
        if (codes->size[i] != src->size[i] || scales->size[i] != src->size[i])
            return fail(MOE_ERR_SHAPE, "codes/scales leading dims must match src");
    if (codes->size[nd - 1] != K / 2 || scales->size[nd - 1] != K / 32)
        return fail(MOE_ERR_SHAPE, "codes must be [.., K/2] and scales [.., K/32]");
    if (codes->stride[nd - 1] != 1 || scales->stride[nd - 1] != 1)
        return fail(MOE_ERR_LAYOUT, "codes and scales need last-dim stride 1");
    if (overlaps(*codes, *src) || overlaps(*scales, *src) || overlaps(*codes, *scales))
        return fail(MOE_ERR_LAYOUT, "outputs overlap");
    QuantParams p{};
    p.src = (const uint16_t*)src->data;
    p.codes = (uint8_t*)codes->data;
    p.scales = (uint8_t*)scales->data;
    p.K = K;
    if (nd == 3) {
        p.E = src->size[0];
        p.R = src->size[1];
        p.ss_e = src->stride[0];
        p.ss_r = src->stride[1];
        p.ss_k = src->stride[2];
        p.cs_e = codes->stride[0];
        p.cs_r = codes->stride[1];
        p.xs_e = scales->stride[0];
        p.xs_r = scales->stride[1];
    } else {
        p.E = 1;
        p.R = src->size[0];
        p.ss_e = 0;
        p.ss_r = src->stride[0];
        p.ss_k = src->stride[1];
        p.cs_e = 0;
        p.cs_r = codes->stride[0];
        p.xs_e = 0;
        p.xs_r = scales->stride[0];
    }
    hipError_t e = launch_quant_mxfp4(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quant_mxfp4");
    return ok();
}

int moe_rmsnorm(const moe_tensor_t* x, const moe_tensor_t* weight, float eps, const moe_tensor_t* out,
                moe_stream_t stream) {
    int rc;
    if ((rc = check_desc(x, "x", MOE_DT_BF16, 2))) return rc;
    const int64_t T = x->size[0], H = x->size[1];
    if ((rc = check_norm_weight(weight, H))) return rc;
    if ((rc = check_desc(out, "out", MOE_DT_BF16, 2))) return rc;
    if ((rc = check_shape(*out, "out", {T, H}))) return rc;
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(MOE_ERR_ARG, "eps must be finite and >= 0");
    if (H < 8 || H % 8 != 0 || H > ((int64_t)1 << 24) || T > ((int64_t)1 << 30))
        return fail(MOE_ERR_UNSUPPORTED, "H = %lld must be a positive multiple of 8 (T = %lld)", (long long)H,
                    (long long)T);
    if (overlaps(*out, *x) || overlaps(*out, *weight)) return fail(MOE_ERR_LAYOUT, "out overlaps an input");
    if (T == 0) return ok();
    NormParams np{};
    norm_params(&np, *x, *weight, eps);
    np.out = (uint16_t*)out->data;
    np.os_t = out->stride[0];
    np.os_h = H > 1 ? out->stride[1] : 1;
    hipError_t e = launch_rmsnorm(np, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm");
    return ok();
}

int moe_combine(const moe_tensor_t* y_rows, const moe_tensor_t* topk_ids, const moe_tensor_t* topk_weights,
                int32_t num_experts, const moe_tensor_t* out, moe_stream_t stream) {
    int rc;
    if ((rc = check_desc(y_rows, "y_rows", MOE_DT_BF16, 3))) return rc;
    const int64_t T = y_rows->size[0], k = y_rows->size[1], H = y_rows->size[2];
    if ((rc = check_desc(topk_ids, "topk_ids", MOE_DT_I32, 2))) return rc;
    if ((rc = check_desc(topk_weights, "topk_weights", MOE_DT_F32, 2))) return rc;
    if ((rc = check_desc(out, "out", MOE_DT_BF16, 2))) return rc;
    if ((rc = check_shape(*topk_ids, "topk_ids", {T, k}))) return rc;
    if ((rc = check_shape(*topk_weights, "topk_weights", {T, k}))) return rc;
    if ((rc = check_shape(*out, "out", {T, H}))) return rc;
    if (num_experts < 1) return fail(MOE_ERR_ARG, "num_experts = %d must be >= 1", num_experts);
    if (k < 1 || k > 64 || H < 4 || H % 4 != 0 || H > (1 << 24) || T > ((int64_t)1 << 24))
        return fail(MOE_ERR_UNSUPPORTED, "k = %lld and H = %lld (a multiple of 4) outside what the library handles",
                    (long long)k, (long long)H);
    const moe_tensor_t& y = *y_rows;
    if (y.stride[2] != 1 || !aligned16(y.data) || (T > 1 && (y.stride[0] * 2) % 16 != 0) ||
        (k > 1 && (y.stride[1] * 2) % 16 != 0))
        return fail(MOE_ERR_LAYOUT, "y_rows: needs last stride 1 and 16-byte aligned rows");
    const moe_tensor_t* ins[3] = {y_rows, topk_ids, topk_weights};
    for (auto* t : ins)
        if (overlaps(*out, *t)) return fail(MOE_ERR_LAYOUT, "out overlaps an input");
    if (T == 0) return ok();
    CombineParams cp{};
    cp.y = (const uint16_t*)y.data;
    cp.ys_t = y.stride[0];
    cp.ys_j = y.stride[1];
    cp.e_off = 0;
    cp.ids = (const int32_t*)topk_ids->data;
    cp.is_t = topk_ids->stride[0];
    cp.is_j = topk_ids->stride[1];
    cp.w = (const float*)topk_weights->data;
    cp.ws_t = topk_weights->stride[0];
    cp.ws_j = topk_weights->stride[1];
    cp.out = (uint16_t*)out->data;
    cp.os_t = out->stride[0];
    cp.os_h = out->stride[1];
    cp.T = (int32_t)T;
    cp.k = (int32_t)k;
    cp.E = num_experts;
    cp.H = (int32_t)H;
    hipError_t e = launch_combine(cp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine");
    return ok();
}

int moe_query_config(const moe_fused_args_t* args, moe_config_t* cfg) {
    if (!cfg) return fail(MOE_ERR_NULL, "cfg is NULL");
    Plan pl;
    int64_t chunk = 0;
    int rc = plan_auto(args, &pl, &chunk);
    if (rc) return rc;
    cfg->bucket = bucket_of(pl.T);
    cfg->block_m = pl.ks[0].bm;
    cfg->block_m2 = pl.ks[1].bm;
    const int base = args->mode == MOE_MODE_MXFP4 ? 10 : 0;
    cfg->gemm1_kernel = pl.small1 ? base + 7 : (pl.ks[0].persist ? base + 9 : base + (pl.ks[0].tile ? 2 : 0) + 1);
    cfg->gemm2_kernel =
        pl.fuse ? base + 6
                : (pl.ks[1].persist ? base + 10
                                    : (pl.ks[1].tile == 7 || pl.ks[1].tile == 8 ? base + 8
                                                                                : base + (pl.ks[1].tile ? 2 : 0) + 2));
    cfg->gemm1_split_k = pl.small1 ? 4 : (pl.ks[0].tile ? 1 : pl.ks[0].wk);
    cfg->gemm2_split_k = pl.fuse ? (base ? 1 : 4) : (pl.ks[1].tile ? 1 : pl.ks[1].wk);
    cfg->config_index = pl.cfg_index;
    cfg->num_configs = kNumConfigs;
    return ok();
}

int moe_fused_workspace_size(const moe_fused_args_t* args, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
    Plan pl;
    int64_t chunk = 0;
    int rc = plan_auto(args, &pl, &chunk);
    if (rc) return rc;
    *bytes = pl.total;
    return ok();
}

int moe_fused_fwd(const moe_fused_args_t* args, void* ws, size_t ws_bytes, moe_stream_t stream) {
    Plan pl;
    int64_t chunk = 0;
    int rc = plan_auto(args, &pl, &chunk);
    if (rc) return rc;
    if (args->x.size[0] == 0) return ok();
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pl.total)
        return fail(MOE_ERR_WORKSPACE, "fused forward needs %zu bytes of 256-byte aligned workspace", pl.total);
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    if (!chunk) return run_fused(*args, pl, base, s);
    // token chunks, each with the configuration of the first (the whole
    // call's bucket); both chunk shapes are planned before any launch
    const int64_t T = args->x.size[0], tail = T % chunk;
    Plan pl_tail;
    if (tail) {
        moe_fused_args_t c = token_slice(*args, T - tail, tail);
        c.force_config = pl.cfg_index;
        if ((rc = plan_fused(&c, &pl_tail))) return rc;
    }
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int64_t n = std::min(chunk, T - t0);
        moe_fused_args_t c = token_slice(*args, t0, n);
        c.force_config = pl.cfg_index;
        if ((rc = run_fused(c, n == chunk ? pl : pl_tail, base, s))) return rc;
    }
    return ok();
}

int moe_fused_bwd_workspace_size(const moe_bwd_args_t* args, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
    BwdPlan pl;
    int rc = plan_bwd(args, &pl);
    if (rc) return rc;
    *bytes = pl.total;
    return ok();
}

int moe_fused_bwd(const moe_bwd_args_t* args, void* ws, size_t ws_bytes, moe_stream_t stream) {
    BwdPlan pl;
    int rc = plan_bwd(args, &pl);
    if (rc) return rc;
    const Plan& f = pl.fwd;
    if (f.T == 0) return ok();
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pl.total)
        return fail(MOE_ERR_WORKSPACE, "backward needs %zu bytes of 256-byte aligned workspace", pl.total);
    const moe_bwd_args_t& b = *args;
    const moe_fused_args_t& a = b.fwd;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    const int64_t T = f.T, H = f.H, I = f.I, E = f.E, k = f.k, A = f.A;
    int32_t* sorted = (int32_t*)(base + pl.off_sorted);
    int32_t* bexp = (int32_t*)(base + pl.off_bexp);
    int32_t* npad = (int32_t*)(base + pl.off_npad);
    int32_t* ebf = (int32_t*)(base + pl.off_ebf);
    int32_t* ebl = (int32_t*)(base + pl.off_ebl);
    float* gu = (float*)(base + pl.off_gu);
    float* q = (float*)(base + pl.off_q);
    uint16_t* dgu = (uint16_t*)(base + pl.off_dgu);
    uint16_t* wh = (uint16_t*)(base + pl.off_wh);
    float* dxa = (float*)(base + pl.off_dxa);
    const int max_blocks = (int)(pl.cap / kBwdBM);
    hipError_t e;

    // align at block_m 64, and each expert's range of sorted blocks
    AlignParams ap{};
    ap.ids = (const int32_t*)a.topk_ids.data;
    ap.is_t = a.topk_ids.stride[0];
    ap.is_j = a.topk_ids.stride[1];
    ap.T = (int32_t)T;
    ap.k = (int32_t)k;
    ap.A = (int32_t)A;
    ap.E = (int32_t)E;
    ap.e_off = f.e_off;
    ap.bm = kBwdBM;
    ap.cap = (int32_t)pl.cap;
    ap.sorted = sorted;
    ap.block_expert = bexp;
    ap.n_padded = npad;
    ap.counts = (int32_t*)(base + pl.off_counts);
    if ((e = launch_align(ap, s)) != hipSuccess) return hip_fail(e, "align");
    if ((e = launch_bwd_expert_blocks(bexp, npad, kBwdBM, max_blocks, ebf, ebl, (int)E, s)) != hipSuccess)
        return hip_fail(e, "expert blocks");

    // activation rows with unit stride and 16-byte alignment
    auto rows_of = [&](const moe_tensor_t& t, bool pack, size_t off, const uint16_t** ptr, int64_t* row) {
        if (!pack) {
            *ptr = (const uint16_t*)t.data;
            *row = t.size[0] > 1 ? t.stride[0] : H;
            return hipSuccess;
        }
        PackParams pp{};
        pp.src = (const uint16_t*)t.data;
        pp.s_t = t.stride[0];
        pp.s_h = t.stride[1];
        pp.dst = (uint16_t*)(base + off);
        pp.T = T;
        pp.H = H;
        *ptr = pp.dst;
        *row = H;
        return launch_pack_bf16(pp, s);
    };
    const uint16_t *xr, *dr;
    int64_t x_row, d_row;
    if ((e = rows_of(a.x, pl.pack_x, pl.off_xp, &xr, &x_row)) != hipSuccess) return hip_fail(e, "pack x");
    if ((e = rows_of(b.dout, pl.pack_d, pl.off_dp, &dr, &d_row)) != hipSuccess) return hip_fail(e, "pack dout");

    const int64_t no_split = (int64_t)1 << 62;
    auto act_src = [&](const uint16_t* p0, int64_t row, int kind) {
        BwdRowSrc r{};
        r.base[0] = r.base[1] = p0;
        r.r_stride[0] = r.r_stride[1] = row;
        r.split = no_split;
        r.kind = kind;
        return r;
    };
    BwdRowSrc w13{};
    w13.base[0] = (const uint16_t*)a.gate.data;
    w13.base[1] = (const uint16_t*)a.up.data;
    w13.e_stride[0] = a.gate.stride[0];
    w13.e_stride[1] = a.up.stride[0];
    w13.r_stride[0] = a.gate.stride[1];
    w13.r_stride[1] = a.up.stride[1];
    w13.split = I;
    w13.kind = 0;
    BwdRowSrc w2s{};
    w2s.base[0] = w2s.base[1] = (const uint16_t*)a.w2.data;
    w2s.e_stride[0] = w2s.e_stride[1] = a.w2.stride[0];
    w2s.r_stride[0] = w2s.r_stride[1] = a.w2.stride[1];
    w2s.split = no_split;
    w2s.kind = 0;
    BwdGemmParams g{};
    g.sorted = sorted;
    g.block_expert = bexp;
    g.n_padded = npad;
    g.eb_first = ebf;
    g.eb_last = ebl;
    g.A = (int32_t)A;
    g.k = (int32_t)k;

    // g | u = x_t [gate_e; up_e]^T, by sorted row blocks
    g.a = act_src(xr, x_row, 1);
    g.b = w13;
    g.K = (int32_t)H;
    g.n_tiles = (int32_t)(2 * I / 128);
    g.rows_out = gu;
    g.rows_ld = 2 * I;
    if ((e = launch_bwd_gemm(0, 0, 0, g, (int64_t)max_blocks * g.n_tiles, s)) != hipSuccess)
        return hip_fail(e, "recompute gemm1");
    // q = dout_t w2_e (K = H, the rows of w2)
    g.a = act_src(dr, d_row, 1);
    g.b = w2s;
    g.K = (int32_t)H;
    g.n_tiles = (int32_t)(I / 128);
    g.rows_out = q;
    g.rows_ld = I;
    if ((e = launch_bwd_gemm(0, 1, 0, g, (int64_t)max_blocks * g.n_tiles, s)) != hipSuccess)
        return hip_fail(e, "dout w2");
    // per slot: dw, dg | du, w hb
    BwdActParams bp{};
    bp.gu = gu;
    bp.q = q;
    bp.dgu = dgu;
    bp.wh = wh;
    bp.ids = (const int32_t*)a.topk_ids.data;
    bp.is_t = a.topk_ids.stride[0];
    bp.is_j = a.topk_ids.stride[1];
    bp.w = (const float*)a.topk_weights.data;
    bp.ws_t = a.topk_weights.stride[0];
    bp.ws_j = a.topk_weights.stride[1];
    bp.dw = (float*)b.dtopk_weights.data;
    bp.dws_t = b.dtopk_weights.stride[0];
    bp.dws_j = b.dtopk_weights.stride[1];
    bp.e_off = f.e_off;
    bp.E = (int32_t)E;
    bp.k = (int32_t)k;
    bp.I = (int32_t)I;
    bp.A = A;
    if ((e = launch_bwd_act(bp, s)) != hipSuccess) return hip_fail(e, "backward activation");
    // per-slot dx = [dg | du] [gate_e; up_e] (K = 2I, the rows of w13)
    g.a = act_src(dgu, 2 * I, 2);
    g.b = w13;
    g.K = (int32_t)(2 * I);
    g.n_tiles = (int32_t)(H / 128);
    g.rows_out = dxa;
    g.rows_ld = H;
    if ((e = launch_bwd_gemm(0, 1, 0, g, (int64_t)max_blocks * g.n_tiles, s)) != hipSuccess)
        return hip_fail(e, "dx gemm");
    // dW2_e = sum over the expert's slots of dout_t (w hb)^T
    g.a = act_src(dr, d_row, 1);
    g.b = act_src(wh, I, 2);
    g.m_tiles = (int32_t)(H / kBwdWgradBM);
    g.n_tiles = (int32_t)(I / 128);
    g.out[0] = g.out[1] = b.dw2.data;
    g.out_e[0] = g.out_e[1] = b.dw2.stride[0];
    g.out_r[0] = g.out_r[1] = b.dw2.stride[1];
    g.out_split = no_split;
    g.out_f32 = pl.wgrad_f32 ? 1 : 0;
    g.out_accumulate = b.accumulate;
    if ((e = launch_bwd_gemm(1, 1, 1, g, E * g.m_tiles * g.n_tiles, s)) != hipSuccess) return hip_fail(e, "dw2 gemm");
    // [dG_e; dU_e] = sum over the expert's slots of [dg; du] x_t^T
    g.a = act_src(dgu, 2 * I, 2);
    g.b = act_src(xr, x_row, 1);
    g.m_tiles = (int32_t)(2 * I / kBwdWgradBM);
    g.n_tiles = (int32_t)(H / 128);
    g.out[0] = b.dgate.data;
    g.out[1] = b.dup.data;
    g.out_e[0] = b.dgate.stride[0];
    g.out_e[1] = b.dup.stride[0];
    g.out_r[0] = b.dgate.stride[1];
    g.out_r[1] = b.dup.stride[1];
    g.out_split = I;
    if ((e = launch_bwd_gemm(1, 1, 1, g, E * g.m_tiles * g.n_tiles, s)) != hipSuccess) return hip_fail(e, "dw13 gemm");
    // dx_t = sum over slots, in order
    BwdDxParams dp{};
    dp.dxa = dxa;
    dp.ids = (const int32_t*)a.topk_ids.data;
    dp.is_t = a.topk_ids.stride[0];
    dp.is_j = a.topk_ids.stride[1];
    dp.e_off = f.e_off;
    dp.E = (int32_t)E;
    dp.k = (int32_t)k;
    dp.T = T;
    dp.H = H;
    dp.dx = (uint16_t*)b.dx.data;
    dp.os_t = b.dx.stride[0];
    dp.os_h = b.dx.stride[1];
    if ((e = launch_bwd_dx(dp, s)) != hipSuccess) return hip_fail(e, "dx combine");
    return ok();
}

}  // extern "C"
