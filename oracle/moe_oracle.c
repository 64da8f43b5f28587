/*
 * CPU oracle for the fused MoE expert-FFN forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the HIP library; it reads the same input bytes
 * through the same strides and computes the plain definition of each step,
 * slowly and in double precision.
 *
 * What is computed, and where it is defined:
 *   route  - softmax over the router logits, top-k, renormalise, with the
 *            weights defined through one stated double-precision exp
 *            (ROCm/aiter PR "TP2 MXFP4 fused-MoE configs for Qwen3.5-397B",
 *            Summary: the unfused 512/10 and shared-expert-fused 513/11
 *            routing conventions; the tiny workload spells out
 *            "softmax -> top-k, renormalised").
 *   align  - the assignments (token t, slot j), flat index a = t*k + j,
 *            grouped by expert in ascending a and each group padded to a
 *            multiple of block_m (aiter PR, Details: the tuner's sorted
 *            token routing and the block_m column of the latency table;
 *            Liger PR #1377, Testing Done: unaligned token tails).
 *   ffn    - for every valid (t, j) with expert e: g = G_e x_t, u = U_e x_t
 *            with gate/up views of the packed w13 [E, 2I, H] addressed by
 *            their real expert stride (Liger PR #1377, Problems and the
 *            review reply on weight_expert_stride), h = SiLU(g) * u
 *            (aiter PR, Details: ActivationType.Silu), y = W2_e h.
 *   combine - out_t = sum_j w_tj * y_tj.
 *   mxfp4  - e2m1 codes with one e8m0 scale per 32 elements along K
 *            (aiter PR, Details: float4_e2m1fn_x2, QuantType.per_1x32) for
 *            weights and activations.
 *   rmsnorm - the row normalisation ahead of the FFN, reading x through
 *            both of its strides in both passes (LightLLM issue #1467,
 *            Summary, Reproduction and Expected Behavior).
 *   backward - the gradients of L = sum over t, n of dout[t, n] * out[t, n]
 *            with respect to x, the top-k weights and the three weight
 *            tensors, by the chain rule through the forward above (Liger PR
 *            #1377, Notes: the grad-enabled path of the same fused MoE).
 *
 * Readings where the pages are silent (each listed with its reason in the
 * design notes): ties in top-k go to the lower expert index and slots are in
 * selection order; the shared expert takes weight 1.0; the MXFP4 scale is
 * floor(log2(amax)) - 2 clamped to [-127, 127] with round-to-nearest-even
 * onto the e2m1 grid, saturating at 6, element 2i in the low nibble; h is
 * rounded to bf16 (bf16 mode) or quantised to MXFP4 per 32 columns (MXFP4
 * mode) from its fp32 value; out is rounded to bf16 once, from fp32.
 *
 * Numbers: products of bf16 or dequantised MXFP4 values are exact in double,
 * sums run sequentially in ascending index order in double. Rounding points
 * that turn a float into a code or a narrower float (h, out) first round the
 * double to fp32, the precision the GPU takes that decision in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EARG (-1)

/* ---------------------------------------------------------------- bf16 */

static double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays NaN. */
static uint16_t orc_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* --------------------------------------------------------------- mxfp4 */

/* The eight magnitudes an e2m1 code can hold (code bits 0..2). */
static const double orc_e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code)
{
    double m = orc_e2m1_mag[code & 7];
    return (code & 8) ? -m : m;
}

/* e8m0 byte -> 2^(byte-127); 255 is NaN. */
double orc_e8m0_value(int byte)
{
    if (byte == 255)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/* Shared exponent of one group: floor(log2(amax)) - 2, clamped to
 * [-127, 127]; a zero group gets -127. amax is an fp32 value. */
static int orc_group_exponent(double amax)
{
    if (amax == 0.0)
        return -127;
    int ex;
    frexp(amax, &ex);            /* amax = m * 2^ex, m in [0.5, 1) */
    int s = (ex - 1) - 2;        /* floor(log2(amax)) - 2 */
    if (s < -127)
        s = -127;
    if (s > 127)
        s = 127;
    return s;
}

/* Nearest e2m1 code to q (already divided by the group scale): search all
 * eight magnitudes; on equal distance the even code wins; anything above 6
 * lands on 6. The sign bit copies the sign of q. */
static int orc_e2m1_nearest(double q)
{
    double a = fabs(q);
    int best = 0;
    double bestd = fabs(a - orc_e2m1_mag[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - orc_e2m1_mag[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best | (signbit(q) ? 8 : 0);
}

/* Quantise n (a multiple of 32) fp32 values to packed codes (n/2 bytes,
 * element 2i in the low nibble) and n/32 scale bytes. */
void orc_mxfp4_quant(const float *v, int64_t n, uint8_t *codes, uint8_t *scales)
{
    for (int64_t g = 0; g < n / 32; ++g) {
        const float *p = v + g * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            double a = fabs((double)p[i]);
            if (a > amax)
                amax = a;
        }
        int s = orc_group_exponent(amax);
        scales[g] = (uint8_t)(s + 127);
        for (int i = 0; i < 32; i += 2) {
            int lo = orc_e2m1_nearest(ldexp((double)p[i], -s));
            int hi = orc_e2m1_nearest(ldexp((double)p[i + 1], -s));
            codes[g * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* Quantise bf16 rows: src[r*rs + c*cs] for r < rows, c < K. */
int orc_mxfp4_quant_bf16(const uint16_t *src, int64_t rows, int64_t K, int64_t rs, int64_t cs,
                         uint8_t *codes, uint8_t *scales)
{
    if (K % 32 != 0)
        return ORC_EARG;
    int err = 0;
    /* rows are independent; threads only split the row loop */
#pragma omp parallel
    {
        float *buf = (float *)malloc(sizeof(float) * (size_t)K);
        if (!buf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < rows; ++r) {
                for (int64_t c = 0; c < K; ++c)
                    buf[c] = (float)orc_bf16_to_double(src[r * rs + c * cs]);
                orc_mxfp4_quant(buf, K, codes + r * (K / 2), scales + r * (K / 32));
            }
        }
        free(buf);
    }
    return err ? ORC_EARG : ORC_OK;
}

/* Dequantise one packed row of K elements. */
static void orc_mxfp4_dequant_row(const uint8_t *codes, const uint8_t *scales, int64_t K, double *out)
{
    for (int64_t c = 0; c < K; ++c) {
        int byte = codes[c / 2];
        int code = (c & 1) ? (byte >> 4) : (byte & 15);
        out[c] = orc_e2m1_value(code) * orc_e8m0_value(scales[c / 32]);
    }
}

/* --------------------------------------------------------------- route */

/*
 * exp(d) in double precision for d <= 0, the exponential the router weights
 * are defined with. The pages fix no exponential, yet routing must match bit
 * for bit, so the weights are defined through one stated sequence of IEEE
 * double operations that any implementation can follow step by step:
 *   d < -708 (or -inf): 0 (every such term is far below what an fp32 weight
 *     can hold next to the leading term 1);
 *   n = rint(d * RN(1/ln 2))                  (ties to even)
 *   r = fma(-n, LN2_HI, d); r = fma(-n, LN2_LO, r)
 *       with LN2_HI = RN(ln 2) and LN2_LO = RN(ln 2 - LN2_HI)
 *   p = 1/13!; p = fma(p, r, 1/i!) for i = 12 down to 0
 *       (Taylor coefficients 1/i!, each the double nearest to it)
 *   result = p * 2^n                          (exact: n >= -1021)
 * Cody-Waite reduction to |r| <= ln2/2 and the degree-13 Taylor polynomial
 * leave a truncation error below 1e-17 relative; the whole sequence is
 * within a few units in the last place of exp(d), which the tests check
 * against math.exp and exact decimal arithmetic.
 */
double orc_route_exp(double d)
{
    static const double inv_ln2 = 0x1.71547652b82fep+0;
    static const double ln2_hi = 0x1.62e42fefa39efp-1;
    static const double ln2_lo = 0x1.abc9e3b39803fp-56;
    if (!(d >= -708.0))
        return 0.0;
    double n = rint(d * inv_ln2);
    double r = fma(-n, ln2_hi, d);
    r = fma(-n, ln2_lo, r);
    double fact = 1.0;
    for (int i = 2; i <= 13; ++i)
        fact *= (double)i;               /* 13! = 6227020800, exact */
    double p = 1.0 / fact;
    for (int i = 12; i >= 0; --i) {
        fact /= (double)(i + 1);         /* i!, exact */
        p = fma(p, r, 1.0 / fact);
    }
    return ldexp(p, (int)n);
}

/*
 * For each token: the k largest logits, one after another, equal logits
 * going to the lower expert index (softmax is strictly increasing, so these
 * are the k largest softmax probabilities; selecting on the logits keeps
 * rounding from creating ties). With m the first pick's logit and
 * e_x = orc_route_exp(l_x - m) in double:
 *   renorm: w_j = fp32(e_j / S), S = ((e_0 + e_1) + ...) + e_{k-1} over the
 *           picks in slot order (the renormalised top-k softmax: the
 *           partition function cancels);
 *   else:   w_j = fp32(e_j / Z), Z = the sum of e_x over all experts in
 *           ascending index order (the plain softmax probability).
 * The double quotient is rounded once to fp32 (nearest, ties to even). With
 * shared_id >= 0 the slot after the k routed ones gets (shared_id, shared_w).
 */
int orc_route(const float *logits, int64_t T, int64_t E, int64_t ls_t, int64_t ls_e, int k,
              int renorm, int shared_id, float shared_w,
              int32_t *ids, int64_t is_t, int64_t is_j, float *w, int64_t ws_t, int64_t ws_j)
{
    if (k <= 0 || k > E)
        return ORC_EARG;
    char *taken = (char *)malloc((size_t)E);
    double *ek = (double *)malloc(sizeof(double) * (size_t)k);
    if (!taken || !ek) {
        free(taken); free(ek);
        return ORC_EARG;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * ls_t;
        memset(taken, 0, (size_t)E);
        double m = 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || row[e * ls_e] > row[best * ls_e])
                    best = e;
            }
            taken[best] = 1;
            ids[t * is_t + j * is_j] = (int32_t)best;
            if (j == 0)
                m = (double)row[best * ls_e];
            ek[j] = orc_route_exp((double)row[best * ls_e] - m);
        }
        double s = 0.0;
        if (renorm) {
            for (int j = 0; j < k; ++j)
                s += ek[j];
        } else {
            for (int64_t e = 0; e < E; ++e)
                s += orc_route_exp((double)row[e * ls_e] - m);
        }
        for (int j = 0; j < k; ++j)
            w[t * ws_t + j * ws_j] = (float)(ek[j] / s);
        if (shared_id >= 0) {
            ids[t * is_t + k * is_j] = shared_id;
            w[t * ws_t + k * ws_j] = shared_w;
        }
    }
    free(taken);
    free(ek);
    return ORC_OK;
}

/* --------------------------------------------------------------- align */

/*
 * sorted[]: for e = 0..E-1, the flat indices a = t*k + j with ids[t, j] == e
 * in ascending a, then the sentinel value A = T*k until the group length is a
 * multiple of bm. block_expert[b] = expert of sorted block b. Ids outside
 * [0, E) are left out. Returns the padded length in *n_padded; fails if it
 * would exceed cap.
 */
int orc_align(const int32_t *ids, int64_t T, int k, int64_t is_t, int64_t is_j, int E, int bm,
              int32_t *sorted, int32_t *block_expert, int64_t cap, int64_t *n_padded)
{
    if (bm <= 0 || k <= 0)
        return ORC_EARG;
    int64_t A = T * (int64_t)k;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        int64_t start = pos;
        for (int64_t a = 0; a < A; ++a) {
            int64_t t = a / k, j = a % k;
            if (ids[t * is_t + j * is_j] == e) {
                if (pos >= cap)
                    return ORC_EARG;
                sorted[pos++] = (int32_t)a;
            }
        }
        while ((pos - start) % bm != 0) {
            if (pos >= cap)
                return ORC_EARG;
            sorted[pos++] = (int32_t)A;
        }
        for (int64_t b = start / bm; b < pos / bm; ++b)
            block_expert[b] = e;
    }
    *n_padded = pos;
    return ORC_OK;
}

/* ----------------------------------------------------------------- ffn */

typedef struct {
    /* mode 0 = bf16, 1 = mxfp4 */
    int32_t mode;
    /* 0: h as computed (double, no rounding); 1: the method's rounding of h
     * (bf16, or MXFP4 quantise + dequantise) */
    int32_t round_h;
    int64_t T, H, I, E, k;
    /* x: bf16 [T, H] */
    const uint16_t *x;
    int64_t xs_t, xs_h;
    /* bf16 weights, element strides: gate/up [E, I, H], w2 [E, H, I] */
    const uint16_t *gate, *up, *w2;
    int64_t gs_e, gs_r, gs_c, us_e, us_r, us_c, w2s_e, w2s_r, w2s_c;
    /* mxfp4 weights: packed codes [E, rows, K/2] and scales [E, rows, K/32],
     * byte strides (expert, row); the last dim is contiguous */
    const uint8_t *gate_q, *up_q, *w2_q, *gate_sc, *up_sc, *w2_sc;
    int64_t gqs_e, gqs_r, uqs_e, uqs_r, w2qs_e, w2qs_r;
    int64_t gss_e, gss_r, uss_e, uss_r, w2ss_e, w2ss_r;
    /* routing */
    const int32_t *ids;
    int64_t is_t, is_j;
    const float *wts;
    int64_t ws_t, ws_j;
} orc_ffn_args;

static double orc_silu_mul(double g, double u)
{
    return g / (1.0 + exp(-g)) * u;
}

/* One token: out_acc[H] = sum_j w_tj * y_tj, with y per the definition. */
static int orc_ffn_token(const orc_ffn_args *a, int64_t t, double *xh, double *wrow, double *hrow,
                         float *hf, uint8_t *hq, uint8_t *hs, double *acc)
{
    const int64_t H = a->H, I = a->I;
    /* x row: exact bf16 value, or MXFP4 quantise + dequantise of it */
    for (int64_t c = 0; c < H; ++c)
        xh[c] = orc_bf16_to_double(a->x[t * a->xs_t + c * a->xs_h]);
    if (a->mode == 1) {
        float *xf = hf; /* reuse: H fp32 scratch is available in hf (size >= H) */
        for (int64_t c = 0; c < H; ++c)
            xf[c] = (float)xh[c];
        uint8_t *xq = hq, *xs = hs;
        orc_mxfp4_quant(xf, H, xq, xs);
        orc_mxfp4_dequant_row(xq, xs, H, xh);
    }
    for (int64_t n = 0; n < H; ++n)
        acc[n] = 0.0;
    for (int64_t j = 0; j < a->k; ++j) {
        int64_t e = a->ids[t * a->is_t + j * a->is_j];
        if (e < 0 || e >= a->E)
            continue;
        double wt = (double)a->wts[t * a->ws_t + j * a->ws_j];
        for (int64_t i = 0; i < I; ++i) {
            double g = 0.0, u = 0.0;
            if (a->mode == 0) {
                const uint16_t *gr = a->gate + e * a->gs_e + i * a->gs_r;
                const uint16_t *ur = a->up + e * a->us_e + i * a->us_r;
                for (int64_t c = 0; c < H; ++c)
                    g += xh[c] * orc_bf16_to_double(gr[c * a->gs_c]);
                for (int64_t c = 0; c < H; ++c)
                    u += xh[c] * orc_bf16_to_double(ur[c * a->us_c]);
            } else {
                orc_mxfp4_dequant_row(a->gate_q + e * a->gqs_e + i * a->gqs_r,
                                      a->gate_sc + e * a->gss_e + i * a->gss_r, H, wrow);
                for (int64_t c = 0; c < H; ++c)
                    g += xh[c] * wrow[c];
                orc_mxfp4_dequant_row(a->up_q + e * a->uqs_e + i * a->uqs_r,
                                      a->up_sc + e * a->uss_e + i * a->uss_r, H, wrow);
                for (int64_t c = 0; c < H; ++c)
                    u += xh[c] * wrow[c];
            }
            hrow[i] = orc_silu_mul(g, u);
        }
        if (a->round_h) {
            if (a->mode == 0) {
                for (int64_t i = 0; i < I; ++i)
                    hrow[i] = orc_bf16_to_double(orc_float_to_bf16((float)hrow[i]));
            } else {
                for (int64_t i = 0; i < I; ++i)
                    hf[i] = (float)hrow[i];
                orc_mxfp4_quant(hf, I, hq, hs);
                orc_mxfp4_dequant_row(hq, hs, I, hrow);
            }
        }
        for (int64_t n = 0; n < H; ++n) {
            double y = 0.0;
            if (a->mode == 0) {
                const uint16_t *wr = a->w2 + e * a->w2s_e + n * a->w2s_r;
                for (int64_t i = 0; i < I; ++i)
                    y += hrow[i] * orc_bf16_to_double(wr[i * a->w2s_c]);
            } else {
                orc_mxfp4_dequant_row(a->w2_q + e * a->w2qs_e + n * a->w2qs_r,
                                      a->w2_sc + e * a->w2ss_e + n * a->w2ss_r, I, wrow);
                for (int64_t i = 0; i < I; ++i)
                    y += hrow[i] * wrow[i];
            }
            acc[n] += wt * y;
        }
    }
    return ORC_OK;
}

/*
 * Forward for the tokens listed in toks[0..n_toks) (all tokens when toks is
 * NULL, n_toks = T). out_acc[r, n] holds the double sum, out_bf16[r, n] its
 * bf16 rounding through fp32. Row r of the outputs is token toks[r].
 */
int orc_ffn(const orc_ffn_args *a, const int64_t *toks, int64_t n_toks, double *out_acc,
            uint16_t *out_bf16)
{
    if (a->mode == 1 && (a->H % 32 != 0 || a->I % 32 != 0))
        return ORC_EARG;
    int64_t wmax = a->H > a->I ? a->H : a->I;
    int err = 0;
#pragma omp parallel
    {
        double *xh = (double *)malloc(sizeof(double) * (size_t)a->H);
        double *wrow = (double *)malloc(sizeof(double) * (size_t)wmax);
        double *hrow = (double *)malloc(sizeof(double) * (size_t)a->I);
        float *hf = (float *)malloc(sizeof(float) * (size_t)wmax);
        uint8_t *hq = (uint8_t *)malloc((size_t)wmax);
        uint8_t *hs = (uint8_t *)malloc((size_t)wmax);
        double *acc = (double *)malloc(sizeof(double) * (size_t)a->H);
        if (!xh || !wrow || !hrow || !hf || !hq || !hs || !acc) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_toks; ++r) {
                int64_t t = toks ? toks[r] : r;
                orc_ffn_token(a, t, xh, wrow, hrow, hf, hq, hs, acc);
                for (int64_t n = 0; n < a->H; ++n) {
                    out_acc[r * a->H + n] = acc[n];
                    out_bf16[r * a->H + n] = orc_float_to_bf16((float)acc[n]);
                }
            }
        }
        free(xh); free(wrow); free(hrow); free(hf); free(hq); free(hs); free(acc);
    }
    return err ? ORC_EARG : ORC_OK;
}

/* ------------------------------------------------------------ backward */

/*
 * Slot quantities of one (token t, expert e) pair in bf16 mode: x row xv[H]
 * and dout row dv[H] as doubles; fills g, u (pre-activations), hb (h with
 * the method's rounding when round_h), q = W2_e^T dout (q_i = sum over n of
 * dout_n W2[n, i]) and returns dL/dw = sum over n of dout_n * y_n with
 * y_n = sum over i of W2[n, i] hb_i.
 */
static double orc_bwd_slot(const orc_ffn_args *a, int64_t e, const double *xv, const double *dv, double *g,
                           double *u, double *hb, double *q)
{
    const int64_t H = a->H, I = a->I;
    for (int64_t i = 0; i < I; ++i) {
        const uint16_t *gr = a->gate + e * a->gs_e + i * a->gs_r;
        const uint16_t *ur = a->up + e * a->us_e + i * a->us_r;
        double gs = 0.0, us = 0.0;
        for (int64_t c = 0; c < H; ++c) {
            gs += xv[c] * orc_bf16_to_double(gr[c * a->gs_c]);
            us += xv[c] * orc_bf16_to_double(ur[c * a->us_c]);
        }
        g[i] = gs;
        u[i] = us;
        double h = orc_silu_mul(gs, us);
        hb[i] = a->round_h ? orc_bf16_to_double(orc_float_to_bf16((float)h)) : h;
        q[i] = 0.0;
    }
    double dw = 0.0;
    for (int64_t n = 0; n < H; ++n) {
        const uint16_t *wr = a->w2 + e * a->w2s_e + n * a->w2s_r;
        double y = 0.0;
        for (int64_t i = 0; i < I; ++i) {
            double wv = orc_bf16_to_double(wr[i * a->w2s_c]);
            y += wv * hb[i];
            q[i] += dv[n] * wv;
        }
        dw += dv[n] * y;
    }
    return dw;
}

/* d SiLU(g) / dg = s (1 + g (1 - s)), s the logistic function of g. */
static double orc_dsilu(double g)
{
    double s = 1.0 / (1.0 + exp(-g));
    return s * (1.0 + g * (1.0 - s));
}

static void orc_row(const uint16_t *p, int64_t s, int64_t n, double *out)
{
    for (int64_t c = 0; c < n; ++c)
        out[c] = orc_bf16_to_double(p[c * s]);
}

/*
 * Backward of the bf16 forward (round_h as in orc_ffn; the pages' grad path
 * uses the same rounding points as the forward it differentiates).
 * For the tokens toks[0..n_toks): dx[r, c] = sum over valid slots j of
 *   sum over i of (dg_i G_e[i, c] + du_i U_e[i, c]), and dw[r, j] = dL/dw_tj
 *   (0 for a skipped slot); dx_bf16 is dx rounded through fp32.
 * For the experts exps[0..n_exps): dgate[m] [I, H], dup[m] [I, H] and
 *   dw2[m] [H, I], summed over every slot routed to the expert in ascending
 *   (t, j): dW2[n, i] += w dout_n hb_i, dG[i, c] += dg_i x_c,
 *   dU[i, c] += du_i x_c,
 * with dh_i = w q_i, dg_i = dh_i u_i SiLU'(g_i), du_i = dh_i SiLU(g_i).
 */
int orc_ffn_bwd(const orc_ffn_args *a, const uint16_t *dout, int64_t ds_t, int64_t ds_h, const int64_t *toks,
                int64_t n_toks, double *dx, uint16_t *dx_bf16, double *dw, const int64_t *exps, int64_t n_exps,
                double *dgate, double *dup, double *dw2)
{
    if (a->mode != 0)
        return ORC_EARG;
    const int64_t H = a->H, I = a->I, k = a->k;
    int err = 0;
#pragma omp parallel
    {
        double *xv = malloc(sizeof(double) * (size_t)H), *dv = malloc(sizeof(double) * (size_t)H);
        double *g = malloc(sizeof(double) * (size_t)I), *u = malloc(sizeof(double) * (size_t)I);
        double *hb = malloc(sizeof(double) * (size_t)I), *q = malloc(sizeof(double) * (size_t)I);
        double *dg = malloc(sizeof(double) * (size_t)I), *du = malloc(sizeof(double) * (size_t)I);
        if (!xv || !dv || !g || !u || !hb || !q || !dg || !du) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_toks; ++r) {
                const int64_t t = toks[r];
                orc_row(a->x + t * a->xs_t, a->xs_h, H, xv);
                orc_row(dout + t * ds_t, ds_h, H, dv);
                double *dxr = dx + r * H;
                for (int64_t c = 0; c < H; ++c)
                    dxr[c] = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    const int64_t e = a->ids[t * a->is_t + j * a->is_j];
                    dw[r * k + j] = 0.0;
                    if (e < 0 || e >= a->E)
                        continue;
                    const double wt = (double)a->wts[t * a->ws_t + j * a->ws_j];
                    dw[r * k + j] = orc_bwd_slot(a, e, xv, dv, g, u, hb, q);
                    for (int64_t i = 0; i < I; ++i) {
                        const double dh = wt * q[i];
                        dg[i] = dh * u[i] * orc_dsilu(g[i]);
                        du[i] = dh * g[i] / (1.0 + exp(-g[i]));
                    }
                    for (int64_t i = 0; i < I; ++i) {
                        const uint16_t *gr = a->gate + e * a->gs_e + i * a->gs_r;
                        const uint16_t *ur = a->up + e * a->us_e + i * a->us_r;
                        for (int64_t c = 0; c < H; ++c)
                            dxr[c] += dg[i] * orc_bf16_to_double(gr[c * a->gs_c]) +
                                      du[i] * orc_bf16_to_double(ur[c * a->us_c]);
                    }
                }
                for (int64_t c = 0; c < H; ++c)
                    dx_bf16[r * H + c] = orc_float_to_bf16((float)dxr[c]);
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t m = 0; m < n_exps; ++m) {
                const int64_t e = exps[m];
                double *dG = dgate + m * I * H, *dU = dup + m * I * H, *dW = dw2 + m * H * I;
                memset(dG, 0, sizeof(double) * (size_t)(I * H));
                memset(dU, 0, sizeof(double) * (size_t)(I * H));
                memset(dW, 0, sizeof(double) * (size_t)(H * I));
                for (int64_t t = 0; t < a->T; ++t) {
                    for (int64_t j = 0; j < k; ++j) {
                        if (a->ids[t * a->is_t + j * a->is_j] != e)
                            continue;
                        const double wt = (double)a->wts[t * a->ws_t + j * a->ws_j];
                        orc_row(a->x + t * a->xs_t, a->xs_h, H, xv);
                        orc_row(dout + t * ds_t, ds_h, H, dv);
                        (void)orc_bwd_slot(a, e, xv, dv, g, u, hb, q);
                        for (int64_t i = 0; i < I; ++i) {
                            const double dh = wt * q[i];
                            dg[i] = dh * u[i] * orc_dsilu(g[i]);
                            du[i] = dh * g[i] / (1.0 + exp(-g[i]));
                        }
                        for (int64_t n = 0; n < H; ++n)
                            for (int64_t i = 0; i < I; ++i)
                                dW[n * I + i] += wt * dv[n] * hb[i];
                        for (int64_t i = 0; i < I; ++i)
                            for (int64_t c = 0; c < H; ++c) {
                                dG[i * H + c] += dg[i] * xv[c];
                                dU[i * H + c] += du[i] * xv[c];
                            }
                    }
                }
            }
        }
        free(xv); free(dv); free(g); free(u); free(hb); free(q); free(dg); free(du);
    }
    return err ? ORC_EARG : ORC_OK;
}

/* ------------------------------------------------------------- rmsnorm */

/*
 * RMSNorm of T rows of H bf16 values, x[t*xs_t + h*xs_h] (LightLLM issue
 * #1467: the mean of squares and the normalisation both read the element
 * through xs_h; its reference scales the normalised row by the weight):
 *   ms_t = (sum over h of x^2) / H, r_t = 1 / sqrt(ms_t + eps),
 *   y = x * r_t * w[h * w_s],
 * in double, sums in ascending h. out_acc[t*H + h] keeps y, out_bf16 its
 * rounding to bf16 through fp32.
 */
int orc_rmsnorm(const uint16_t *x, int64_t T, int64_t H, int64_t xs_t, int64_t xs_h, const double *w,
                int64_t w_s, double eps, double *out_acc, uint16_t *out_bf16)
{
    if (H < 1 || eps < 0.0)
        return ORC_EARG;
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double v = orc_bf16_to_double(x[t * xs_t + h * xs_h]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t h = 0; h < H; ++h) {
            double y = orc_bf16_to_double(x[t * xs_t + h * xs_h]) * r * w[h * w_s];
            out_acc[t * H + h] = y;
            out_bf16[t * H + h] = orc_float_to_bf16((float)y);
        }
    }
    return ORC_OK;
}

/* Size of orc_ffn_args, so the Python side can check its mirror. */
int64_t orc_ffn_args_size(void) { return (int64_t)sizeof(orc_ffn_args); }
