/*
 * moeffn — fused mixture-of-experts expert-FFN forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The forward pass of one MoE layer, as the pages describe it:
 *   1. route     top-k over the router's softmax, renormalised
 *                (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for
 *                Qwen3.5-397B", Summary: unfused 512/10 and
 *                shared-expert-fused 513/11 routing);
 *   2. align     the (token, slot) assignments grouped by expert, each group
 *                padded to block_m rows (aiter PR, Details: sorted routing
 *                and the block_m column of the tuned latency table);
 *   3. gemm1     gathered token rows x gate_e^T and x up_e^T, where gate and
 *                up may be views into one packed w13 [E, 2I, H] whose expert
 *                stride is 2*I*H (Liger-Kernel PR #1377 "Support strided
 *                Liger MoE input weights", Problems);
 *   4. act       h = SiLU(gate) * up (aiter PR, Details: ActivationType.Silu);
 *   5. gemm2     h x w2_e^T with w2 [E, H, I];
 *   6. combine   out_t = sum over slots j of w_tj * y_tj.
 * bf16 mode runs all of it in bf16 with fp32 accumulation; MXFP4 mode holds
 * weights and activations as e2m1 codes with one e8m0 scale per 32 elements
 * along K (aiter PR, Details: float4_e2m1fn_x2, QuantType.per_1x32).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensors are described by moe_tensor_t: `data` is the device address of
 *   element [0, ..., 0] of the view (any storage offset already applied),
 *   `size`/`stride` are per dimension, strides in elements of `dtype`
 *   (MOE_DT_FP4X2: one element = one byte holding two e2m1 codes, element 2i
 *   of the logical row in the low nibble). Strides may be any positive value;
 *   a dimension of size 1 may have any stride. A packed w13 view, a per-layer
 *   routed_experts slice with token stride L*k (prime-rl PR #2860, Problem)
 *   and an activation with last-dim stride != 1 (LightLLM issue #1467) are all
 *   accepted without copies and give results bit-identical to contiguous
 *   inputs. A layout the kernels cannot read correctly is rejected with
 *   MOE_ERR_LAYOUT, never read as if it were contiguous.
 * - The caller owns all memory: inputs, outputs and the workspace. The
 *   library allocates nothing, keeps no per-call state, performs no host
 *   synchronisation and no device-to-host copy, and launches only on the
 *   caller's stream. Calls are asynchronous and can be captured in a HIP
 *   graph. Two calls that share a workspace must be ordered on one stream.
 * - Every argument check runs on the host before the first launch: a call
 *   that returns an error has enqueued nothing. MOE_ERR_HIP reports a failed
 *   launch; moe_last_error() then holds the HIP error text.
 * - Inputs must be finite (logits may be -inf as long as each row keeps at
 *   least k finite entries). Outputs must not overlap inputs.
 */
#ifndef MOEFFN_H
#define MOEFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_DIMS 4
/* Number of timed stages of moe_fused_fwd (see moe_fused_args_t). */
#define MOE_NUM_STAGES 5

typedef enum {
    MOE_DT_BF16 = 1,   /* bfloat16 */
    MOE_DT_F32 = 2,    /* float32 */
    MOE_DT_I32 = 3,    /* int32 */
    MOE_DT_FP4X2 = 4,  /* two e2m1 codes per byte, element 2i in the low nibble */
    MOE_DT_E8M0 = 5    /* one unsigned byte b per 32 elements, scale 2^(b-127) */
} moe_dtype_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* sizes disagree (e.g. gate H != x H) */
    MOE_ERR_DTYPE = -3,       /* wrong element type for this argument */
    MOE_ERR_LAYOUT = -4,      /* strides or alignment the kernels cannot honour */
    MOE_ERR_WORKSPACE = -5,   /* workspace NULL, misaligned or too small */
    MOE_ERR_UNSUPPORTED = -6, /* sizes outside what the library handles */
    MOE_ERR_HIP = -7,         /* a HIP launch failed */
    MOE_ERR_ARG = -8          /* any other invalid scalar argument */
} moe_status_t;

typedef enum { MOE_MODE_BF16 = 0, MOE_MODE_MXFP4 = 1 } moe_mode_t;
typedef enum { MOE_ACT_SILU = 0 } moe_activation_t;

typedef struct {
    void *data;
    int32_t dtype;                 /* moe_dtype_t */
    int32_t ndim;
    int64_t size[MOE_MAX_DIMS];
    int64_t stride[MOE_MAX_DIMS];  /* in elements */
} moe_tensor_t;

/* A HIP stream (hipStream_t); NULL is the default stream. */
typedef void *moe_stream_t;

/* -------------------------------------------------------------- route --
 * moe_topk_softmax: router, step 1.
 *   logits   [T, E_r] float32, any strides.
 *   k        routed slots, 1 <= k <= min(E_r, 32).
 *   renorm   1: w_j = softmax_j / sum over the k picked (the pages' "top-k,
 *            renormalised"); 0: plain softmax values of the picked experts.
 *   shared_id, shared_w   if shared_id >= 0, slot k is (shared_id, shared_w)
 *            (the 513/11 convention: expert 512 in every token's 11th slot).
 *   ids      [T, k (+1 if shared)] int32 out, any strides.
 *   weights  [T, k (+1)] float32 out, any strides.
 * Picks the k largest logits, ties to the lower expert index, slots in that
 * order. Weight w_j = fp32(e_j / S), rounded once, with e_j = exp(l_j - l_max)
 * in double precision and S the sum of the picked e_j in slot order
 * (renorm) or of all E of them in ascending expert order (plain softmax).
 * The exponential is a stated sequence, so the weights are reproducible bit
 * for bit: n = rint(d * 0x1.71547652b82fep+0) (1/ln2 rounded to double),
 * r = fma(-n, 0x1.62e42fefa39efp-1, d), then r = fma(-n,
 * 0x1.abc9e3b39803fp-56, r) (ln2 split in two doubles), e^r by its degree-13
 * Taylor polynomial in Horner form with fma (coefficients the doubles
 * nearest 1/i!), times 2^n; 0 for d below -708.
 * T = 0 is a no-op.
 */
int moe_topk_softmax(const moe_tensor_t *logits, int32_t k, int32_t renorm, int32_t shared_id,
                     float shared_w, const moe_tensor_t *ids, const moe_tensor_t *weights,
                     moe_stream_t stream);

/* -------------------------------------------------------------- align --
 * moe_align: step 2, standalone.
 *   ids           [T, k] int32, any strides. Ids outside [0, E) are skipped.
 *   num_experts   E >= 1.
 *   block_m       16, 32, 64, 128 or 256.
 *   sorted_ids    [cap] int32 out, contiguous: for e = 0..E-1 the flat
 *                 indices a = t*k + j with ids[t, j] == e in ascending a, then
 *                 the sentinel T*k until the group is a multiple of block_m.
 *                 cap must be >= moe_align_capacity(T*k, E, block_m).
 *   block_expert  [cap / block_m] int32 out: expert of each sorted block.
 *   n_padded      [1] int32 out: used length of sorted_ids.
 *   ws, ws_bytes  scratch of at least moe_align_workspace_size() bytes,
 *                 256-byte aligned.
 * Entries of sorted_ids and block_expert past n_padded are left unspecified.
 */
int moe_align(const moe_tensor_t *ids, int32_t num_experts, int32_t block_m,
              const moe_tensor_t *sorted_ids, const moe_tensor_t *block_expert,
              const moe_tensor_t *n_padded, void *ws, size_t ws_bytes, moe_stream_t stream);
/* Upper bound on n_padded for A assignments. Host only. */
int64_t moe_align_capacity(int64_t assignments, int32_t num_experts, int32_t block_m);
/* Scratch bytes moe_align needs. Host only, no device calls. */
int moe_align_workspace_size(int64_t tokens, int32_t k, int32_t num_experts, int32_t block_m,
                             size_t *bytes);

/* -------------------------------------------------------------- quant --
 * moe_quant_mxfp4: bf16 -> MXFP4, the activation quantisation of step 3 in
 * MXFP4 mode and the offline weight quantisation.
 *   src     [R, K] or [E, R, K] bf16, any strides; K a multiple of 32.
 *   codes   same leading shape, [.., K/2] FP4X2 out; last stride 1.
 *   scales  same leading shape, [.., K/32] E8M0 out; last stride 1.
 * Per group of 32 along K: s = floor(log2(max|v|)) - 2 clamped to
 * [-127, 127] (s = -127 for an all-zero group), scale byte s + 127, each
 * element the e2m1 code nearest to v / 2^s, ties to the even code, saturating
 * at +-6, sign kept (including -0).
 */
int moe_quant_mxfp4(const moe_tensor_t *src, const moe_tensor_t *codes,
                    const moe_tensor_t *scales, moe_stream_t stream);

/* -------------------------------------------------------------- fused --
 * Arguments of the fused forward (steps 2-6).
 *   mode        MOE_MODE_BF16 or MOE_MODE_MXFP4.
 *   activation  MOE_ACT_SILU.
 *   x           [T, H] bf16, any strides (quantised inside in MXFP4 mode).
 *   gate, up    bf16 [E, I, H] | FP4X2 [E, I, H/2]; last stride 1; expert
 *               and row strides free (64-bit), so views into a packed
 *               w13 [E, 2I, H] work as they are.
 *   gate_scale, up_scale   MXFP4 only: E8M0 [E, I, H/32], last stride 1.
 *   w2          bf16 [E, H, I] | FP4X2 [E, H, I/2]; last stride 1.
 *   w2_scale    MXFP4 only: E8M0 [E, H, I/32], last stride 1.
 *   topk_ids    [T, k] int32, any strides. Expert ids are global: the
 *               weights hold experts expert_offset .. expert_offset + E - 1,
 *               and a slot whose id lies outside that range is skipped.
 *   topk_weights [T, k] float32, any strides.
 *   out         [T, H] bf16 out, any strides; ignored when y_rows is given.
 *   stage_events NULL, or 2*MOE_NUM_STAGES hipEvent_t handles created by the
 *               caller; event 2s is recorded before stage s and 2s+1 after
 *               it, on the call's stream; NULL entries are skipped. Stages:
 *               0 align (its launch also prepares the activation: RMSNorm,
 *               MXFP4 quantisation or the re-layout of a strided x), 1
 *               prepare (the RMSNorm of a re-laid-out x, or of the rows of a
 *               per-slot gemm1 that does not fold it in; usually empty),
 *               2 gemm1 + act, 3 gemm2, 4 combine.
 *   force_config  -1 for the built-in choice, else an index into the
 *               library's config list (tests of tile invariance).
 * Numerics: fp32 accumulation; h rounded to bf16 (bf16 mode) or quantised to
 * MXFP4 per 32 columns (MXFP4 mode); per-slot results y rounded to bf16
 * (RNE) in both modes; combine acc = fmaf(w_tj, y_tj, acc) over j = 0..k-1 in
 * slot order from +0 with y widened exactly to fp32, then one round to bf16.
 * The tile configuration depends only on (mode, T, H, I, k) and the global
 * expert count, never on strides, so every layout runs the same arithmetic.
 * For a few tokens a configuration may skip the align (gemm1 per slot, the
 * expert read from topk_ids) and fold the combine into gemm2; the stages it
 * skips are empty (their events are still recorded), and the results are
 * bit-identical to the aligned path with the same K split. Such configurations never write
 * y_rows: with y_rows the built-in choice falls back to the aligned path.
 */
typedef struct {
    int32_t mode;
    int32_t activation;
    moe_tensor_t x;
    moe_tensor_t gate, up;
    moe_tensor_t gate_scale, up_scale;
    moe_tensor_t w2, w2_scale;
    moe_tensor_t topk_ids;
    moe_tensor_t topk_weights;
    moe_tensor_t out;
    void *const *stage_events;
    int32_t force_config;
    /* Expert-parallel shard (Liger-Kernel PR #1377, Notes: the expert-
     * parallel path; one GPU here holds one shard):
     *   expert_offset       global id of the first local expert, >= 0.
     *   num_global_experts  experts over all shards (0: E); it only sizes
     *                       the tile choice, which then matches the
     *                       unsharded call (same K order, same bits).
     *   y_rows              data NULL: combine into out. Otherwise [T, k, H]
     *                       bf16 out with stride(0) == k * stride(1), last
     *                       stride 1, 16-byte aligned rows: row (t, j) gets
     *                       the per-slot result y_tj (bf16) of every local
     *                       slot, other rows are left untouched, and out is
     *                       not written. Every shard can write its slots into
     *                       one buffer (rows sent home); moe_combine then
     *                       gives the unsharded call's out, bit for bit. */
    int32_t expert_offset;
    moe_tensor_t y_rows;
    int32_t num_global_experts;
    /* RMSNorm pre-pass (LightLLM issue #1467, Summary: both passes read x
     * through its strides): norm_weight data NULL: x goes to gemm1 as it is.
     * Otherwise [H] bf16 or float32, any stride, and gemm1 (and, in MXFP4
     * mode, the activation quantisation) reads moe_rmsnorm(x, norm_weight,
     * norm_eps) instead of x; the result is bit-identical to calling
     * moe_rmsnorm first and passing its output as x. */
    float norm_eps;
    moe_tensor_t norm_weight;
} moe_fused_args_t;

/* The tile configuration a call would use. */
typedef struct {
    int32_t bucket;        /* smallest power of two >= T, capped at 32768 */
    int32_t block_m;       /* rows per sorted block of gemm1 */
    int32_t gemm1_kernel;  /* kernel family of gemm1: 1 bf16 weight-streaming, 3 bf16 LDS-tiled,
                              7 bf16 per slot without the align (few tokens; K split 4,
                              bit-identical to 1 with that split); 11, 13 and 17 the same three in
                              MXFP4 mode; 19 MXFP4 weight-streaming as a persistent kernel (one
                              workgroup per compute unit walking its row-block x column-tile items
                              with the weight loads running on from one item into the next;
                              bit-identical to 11) */
    int32_t gemm2_kernel;  /* kernel family of gemm2: gemm1's plus one, or 6 / 16: gemm2 with the
                              combine folded in (few tokens; bf16 with I a multiple of 256 from 512
                              to 1536 and K split 4, MXFP4 with I = 512; bit-identical results),
                              or 18: MXFP4 gemm2 with K = 512 keeping each block's h rows in
                              registers and walking 128-column weight tiles (many tokens;
                              bit-identical results; y rows below 4 GB, else the LDS tile), or 20:
                              MXFP4 gemm2 with K = 512 as a persistent weight stream (see 19;
                              bit-identical results) */
    int32_t gemm1_split_k; /* waves splitting K inside a workgroup */
    int32_t gemm2_split_k;
    int32_t config_index;  /* index into the library's config list */
    int32_t num_configs;   /* size of that list */
    int32_t block_m2;      /* rows per sorted block of gemm2 (a second align when it differs) */
} moe_config_t;

/* Validate args and report the configuration. Host only. */
int moe_query_config(const moe_fused_args_t *args, moe_config_t *cfg);
/* Validate args and report the workspace bytes moe_fused_fwd needs. Host only. */
int moe_fused_workspace_size(const moe_fused_args_t *args, size_t *bytes);
/* The fused forward: align, (prepare), gemm1 + act, gemm2, combine (or the
 * y_rows output).
 * ws: caller-owned device scratch, 256-byte aligned, >= the reported size;
 * its contents on entry do not matter. T = 0 returns MOE_OK with no launch. */
int moe_fused_fwd(const moe_fused_args_t *args, void *ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------ no allocation --
 * moe_fused_fwd_noalloc: moe_fused_fwd for callers that cannot allocate
 * device memory or bring a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *   args, stream  exactly as for moe_fused_fwd (same checks, kernels and
 *                 results, bit for bit); stream must belong to the current
 *                 device.
 * The workspace is the library's own device array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB), which every GPU the library runs on
 * holds from the first call until the process ends. The call allocates
 * nothing and calls no allocating routine. A call whose
 * moe_fused_workspace_size exceeds that size returns MOE_ERR_WORKSPACE
 * before any launch (for the Qwen3-235B-shaped bf16 layer that is beyond
 * about 600 tokens; the few-token configurations need a few KB). Every call
 * on one GPU shares that GPU's array: calls that overlap there (other
 * streams, other host threads) race, so callers order them.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_fused_fwd_noalloc(const moe_fused_args_t *args, moe_stream_t stream);

/* ----------------------------------------------------------- backward --
 * moe_fused_bwd: gradients of L = sum over t, n of dout[t, n] * out[t, n]
 * for the bf16 forward (Liger-Kernel PR #1377, Notes: the grad-enabled path
 * of the same fused MoE; here it takes the same strided inputs as the
 * forward, packed w13 views included).
 *   fwd          the forward's arguments. mode MOE_MODE_BF16; out is not
 *                written (give dx's descriptor or leave it empty);
 *                expert_offset works as in the forward; y_rows and
 *                norm_weight must be empty (MOE_ERR_UNSUPPORTED otherwise).
 *   dout         [T, H] bf16, any strides.
 *   dx           [T, H] bf16 out, any strides.
 *   dgate, dup   [E, I, H] out, float32 or bf16, last stride 1, expert and row
 *                strides free (views of one packed dw13 [E, 2I, H] work),
 *                rows 16-byte (f32) or 8-byte (bf16) aligned.
 *   dw2          [E, H, I] out, same rules.
 *   dtopk_weights [T, k] float32 out, any strides: dL/dw_tj, 0 for a
 *                skipped slot.
 *   accumulate   0: dgate, dup, dw2 are overwritten (zeros for an expert
 *                without slots). 1: this call's gradients are added to
 *                them (g = g + new in fp32, rounded once for bf16) and
 *                experts without slots are left untouched, as when
 *                gradients accumulate over micro-batches. dx and
 *                dtopk_weights are always overwritten.
 * Per slot (t, j) of expert e, with g, u, h and its bf16 rounding hb exactly
 * as the forward computes them (g, u recomputed): q = w2_e^T dout_t,
 * dw_tj = <q, hb>, dh = w_tj q, dg = dh u SiLU'(g), du = dh SiLU(g); dg, du
 * and w_tj hb are rounded to bf16 before the GEMMs that use them. dx_t sums
 * the slots in order in fp32; each weight gradient sums its expert's slots in
 * sorted (t, j) order in fp32. Sizes: H and I multiples of 128. Every check
 * runs before the first launch; the workspace is the caller's.
 */
typedef struct {
    moe_fused_args_t fwd;
    moe_tensor_t dout;
    moe_tensor_t dx;
    moe_tensor_t dgate, dup;
    moe_tensor_t dw2;
    moe_tensor_t dtopk_weights;
    int32_t accumulate;
    int32_t reserved;
} moe_bwd_args_t;

/* Validate args and report the workspace bytes moe_fused_bwd needs. Host only. */
int moe_fused_bwd_workspace_size(const moe_bwd_args_t *args, size_t *bytes);
int moe_fused_bwd(const moe_bwd_args_t *args, void *ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------ rmsnorm --
 * moe_rmsnorm: the RMSNorm ahead of the expert FFN (LightLLM issue #1467,
 * Summary and Expected Behavior).
 *   x       [T, H] bf16, any strides; H a multiple of 8.
 *   weight  [H] bf16 or float32, any stride.
 *   eps     >= 0, added to the mean of squares.
 *   out     [T, H] bf16 out, any strides, not overlapping x or weight.
 * out[t, h] = bf16_RNE((x[t, h] * r_t) * weight[h]) in fp32, with
 * r_t = 1 / sqrt(ss_t / H + eps) and ss_t the fp32 sum of x[t, h]^2 in one
 * fixed order (64 partial fmaf chains over 8-element chunks c = q, q + 64,
 * ..., then a 64-way pairwise tree), the same for every layout of x and out,
 * so strided and contiguous inputs give identical bits. T = 0 is a no-op.
 */
int moe_rmsnorm(const moe_tensor_t *x, const moe_tensor_t *weight, float eps, const moe_tensor_t *out,
                moe_stream_t stream);

/* ------------------------------------------------------------ combine --
 * moe_combine: step 6 on its own, for per-slot results computed elsewhere
 * (the rows y_rows of expert-parallel shards, sent back to the tokens' home).
 *   y_rows        [T, k, H] bf16, last stride 1, 16-byte aligned rows.
 *   topk_ids      [T, k] int32, any strides: slot (t, j) counts when
 *                 0 <= id < num_experts (global ids), else it is skipped and
 *                 its row is not read.
 *   topk_weights  [T, k] float32, any strides.
 *   out           [T, H] bf16 out, any strides.
 * out_t = bf16(acc), acc = fmaf(w_tj, y_tj, acc) over counted j in slot
 * order from +0, exactly the fused call's combine. T = 0 is a no-op.
 */
int moe_combine(const moe_tensor_t *y_rows, const moe_tensor_t *topk_ids,
                const moe_tensor_t *topk_weights, int32_t num_experts, const moe_tensor_t *out,
                moe_stream_t stream);

/* ------------------------------------------------------------- errors --
 * Static text for a status code; never NULL. */
const char *moe_strerror(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOEFFN_H */
