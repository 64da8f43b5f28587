// Persistent weight-streaming GEMMs (MXFP4): one workgroup per compute unit
// walks a static list of work items and keeps its waves' weight rings full
// from one item into the next. Same parameter block, operand layouts and
// MFMA sequence as the per-tile weight streams in gemm_stream.hip, so the
// results are bit-identical to theirs.
#pragma once

#include "moe_internal.h"

namespace moe {

// gemm1 + SiLU(gate) * up with h quantised to MXFP4 (stage 1 only):
// bm 16 or 32 rows per sorted block with nw 4 or 8 waves per workgroup (32 h
// columns each), or bm 64 with 4 waves. Needs K in {2048, 4096} (and 8192
// with 4 waves and bm up to 32: the scale runs of two items sit in LDS) and
// N % (32 * nw) == 0.
bool gemm1_persist_supported(int bm, int nw, int64_t K, int64_t N);
hipError_t launch_gemm1_persist(int bm, int nw, const GemmParams& p, hipStream_t s);

// gemm2 (y rows by flat assignment, bf16) with K = 512 exactly: bm 16, 32 or
// 64, four waves of 64 output columns, N % 256 == 0.
bool gemm2_persist_supported(int bm, int64_t K, int64_t N);
hipError_t launch_gemm2_persist(int bm, const GemmParams& p, hipStream_t s);

}  // namespace moe
