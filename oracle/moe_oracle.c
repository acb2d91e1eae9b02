/*
 * moe_oracle.c -- CPU oracle for the forward pass of a sparse
 * Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library
 * never links, includes or calls it, and this file includes nothing from
 * the GPU side: the two share no code.
 *
 * What it computes follows the page "Mixture of experts" (rayaq.ca,
 * ml-models/mixture-of-experts), section Mechanics:
 *   - "Replacing the feed-forward block": h = W_r x, p = softmax(h),
 *     y = sum over i in TopK(h) of g_i(x) * E_i(x);
 *   - "Top-k gating": the Switch gate (g = full-softmax p of the argmax
 *     expert) and the renormalised top-k gate (softmax over the k chosen
 *     logits); noise, when used, is added to the logits before the top-k;
 *   - "The load-balancing loss": f_i, P_i, E * sum f_i P_i, and the ST-MoE
 *     z statistic mean_t (log sum_j exp h_tj)^2;
 *   - "Capacity and dropped tokens": capacity from the capacity factor,
 *     slots filled in token (position) order, overflow tokens skip the
 *     expert and contribute nothing to the layer output;
 * and section Implementation (the SwiGLU expert, bias-free Linears, the
 * float32 router, the token-ordered per-expert lists).
 *
 * Precision: every input is fp32 (bf16 inputs are widened exactly by the
 * caller).  Every sum is accumulated in double, sequentially, in index
 * order, and rounded to fp32 once where a stored fp32 tensor is produced
 * (logits, expert hidden H, expert output rows, layer output).  Threads
 * split tokens or rows only, never a sum, so results do not depend on the
 * thread count.  The one blocking used (several independent output
 * elements updated in the same inner loop) keeps each element's own sum
 * strictly sequential; it only lets the compiler vectorise across
 * independent elements.
 *
 * Readings of points the page leaves open (each is also listed in the
 * design notes of the repository):
 *   - noise and bias are added to the logits, and the noisy logits are
 *     used everywhere downstream (p, top-k, gates, statistics);
 *   - top-k order: descending logit, ties to the lower expert index;
 *   - capacity C = ceil(cf * T * k / E) evaluated in double in exactly
 *     that order; cf <= 0 means no limit;
 *   - drop priority is token order within each expert, whatever the slot;
 *   - gates are not renormalised after drops;
 *   - f_i counts top (slot-0) choices before any drop;
 *   - GELU is the exact erf form;
 *   - shared experts (section "Total versus active parameters") have the
 *     routed experts' shape and activation, no gate, and run on every
 *     token, dropped ones included; the layer output then adds the block's
 *     residual: y = res + routed + shared.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GATE_RENORM 0 /* softmax over the k selected logits */
#define ORC_GATE_SWITCH 1 /* full-softmax probability of each selected expert */

#define ORC_ACT_RELU 0
#define ORC_ACT_GELU 1
#define ORC_ACT_SWIGLU 2

/* Number of independent output elements updated together in one inner loop. */
#define ORC_BLK 8

/*
 * Router logits ("Replacing the feed-forward block": h = W_r x; the
 * router is one bias-free Linear with E rows, computed in float32 per the
 * Implementation section's closing advice).
 *   x     [T][d]   fp32
 *   Wr    [E][d]   fp32
 *   bias  [E]      fp32 or NULL
 *   noise [T][E]   fp32 or NULL ("Top-k gating": noise added to the logits
 *                  before the top-k)
 *   h     [T][E]   fp32 out: h[t][i] = fl32(sum_j x[t][j] Wr[i][j] + b[i] + n[t][i])
 */
void orc_router_logits(int64_t T, int64_t d, int64_t E, const float *x,
                       const float *Wr, const float *bias, const float *noise,
                       float *h)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *xt = x + t * d;
        for (int64_t i = 0; i < E; ++i) {
            const float *wi = Wr + i * d;
            double acc = 0.0;
            for (int64_t j = 0; j < d; ++j)
                acc += (double)xt[j] * (double)wi[j];
            if (bias)
                acc += (double)bias[i];
            if (noise)
                acc += (double)noise[t * E + i];
            h[t * E + i] = (float)acc;
        }
    }
}

/*
 * Softmax, log-sum-exp, top-k and gates for every token.
 *   h      [T][E] fp32 logits
 *   idx    [T][k] int32 out: the k largest logits, largest first, ties to
 *                 the lower expert index ("Top-k gating": keep the k
 *                 largest logits)
 *   gates  [T][k] double out:
 *                 RENORM: softmax over the k selected logits
 *                 SWITCH: full-softmax probability p of each selected expert
 *   p      [T][E] double out (may be NULL): p = softmax(h)
 *   lse    [T]    double out (may be NULL): log sum_j exp h_j
 * Returns 0, or -1 on bad arguments.
 */
int orc_gate(int64_t T, int64_t E, int64_t k, int mode, const float *h,
             int32_t *idx, double *gates, double *p, double *lse)
{
    if (k < 1 || k > E || (mode != ORC_GATE_RENORM && mode != ORC_GATE_SWITCH))
        return -1;
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
    /* per-thread mark of the experts already taken, reset for every token */
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        bad = 1;
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        if (!taken)
            continue;
        const float *ht = h + t * E;
        /* full softmax in double */
        double m = (double)ht[0];
        for (int64_t i = 1; i < E; ++i)
            if ((double)ht[i] > m)
                m = (double)ht[i];
        double s = 0.0;
        for (int64_t i = 0; i < E; ++i)
            s += exp((double)ht[i] - m);
        if (p)
            for (int64_t i = 0; i < E; ++i)
                p[t * E + i] = exp((double)ht[i] - m) / s;
        if (lse)
            lse[t] = m + log(s);

        /* top-k by k successive scans for the best expert not yet taken;
         * the strict '>' on an ascending scan keeps the lower index on a tie */
        memset(taken, 0, (size_t)E);
        int32_t *it = idx + t * k;
        for (int64_t sl = 0; sl < k; ++sl) {
            int64_t best = -1;
            for (int64_t i = 0; i < E; ++i)
                if (!taken[i] && (best < 0 || ht[i] > ht[best]))
                    best = i;
            taken[best] = 1;
            it[sl] = (int32_t)best;
        }

        double *gt = gates + t * k;
        if (mode == ORC_GATE_RENORM) {
            /* softmax over the selected logits, shifted by the largest one */
            double top = (double)ht[it[0]];
            double den = 0.0;
            for (int64_t sl = 0; sl < k; ++sl)
                den += exp((double)ht[it[sl]] - top);
            for (int64_t sl = 0; sl < k; ++sl)
                gt[sl] = exp((double)ht[it[sl]] - top) / den;
        } else {
            for (int64_t sl = 0; sl < k; ++sl)
                gt[sl] = exp((double)ht[it[sl]] - m) / s;
        }
    }
    free(taken);
    }
    return bad ? -1 : 0;
}

/*
 * Expert capacity ("Capacity and dropped tokens": tokens per batch over
 * number of experts, times the capacity factor).  With k slots per token
 * the assignments per batch are T*k, which is what a factor of 1 must
 * balance exactly; the result is rounded up.  cf <= 0 means no limit
 * (dropless), returned as -1.
 */
int64_t orc_capacity(int64_t T, int64_t E, int64_t k, double cf)
{
    if (!(cf > 0.0))
        return -1;
    return (int64_t)ceil(cf * (double)T * (double)k / (double)E);
}

/*
 * Dispatch with capacity ("Capacity and dropped tokens"; the Implementation
 * listing's per-expert token lists, which are in token order and cut at
 * the capacity).  For each expert e, its assignments (t, s) with
 * idx[t][s] == e are ranked in token order; rank < C is kept, the rest
 * are dropped.  Kept rows are laid out expert after expert.
 *   idx          [T][k] int32 in
 *   C            capacity, or < 0 for no limit
 *   routed       [E]    out: assignments per expert before dropping
 *   kept         [E]    out: min(routed, C)
 *   offsets      [E+1]  out: exclusive prefix sum of kept
 *   row_of_slot  [T][k] out: row of the kept assignment, -1 if dropped
 *   token_of_row [T*k]  out: token of each kept row (first offsets[E] valid;
 *                       the rest are set to -1)
 *   dropped      [T][k] out: 1 if dropped, else 0
 */
void orc_dispatch(int64_t T, int64_t E, int64_t k, int64_t C,
                  const int32_t *idx, int32_t *routed, int32_t *kept,
                  int32_t *offsets, int32_t *row_of_slot,
                  int32_t *token_of_row, uint8_t *dropped)
{
    for (int64_t e = 0; e < E; ++e) {
        int64_t n = 0;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t s = 0; s < k; ++s)
                if (idx[t * k + s] == e)
                    ++n;
        routed[e] = (int32_t)n;
        kept[e] = (int32_t)((C >= 0 && n > C) ? C : n);
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + kept[e];
    for (int64_t r = 0; r < T * k; ++r)
        token_of_row[r] = -1;
    for (int64_t e = 0; e < E; ++e) {
        int64_t rank = 0;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t s = 0; s < k; ++s) {
                if (idx[t * k + s] != e)
                    continue;
                if (C < 0 || rank < C) {
                    int32_t row = offsets[e] + (int32_t)rank;
                    token_of_row[row] = (int32_t)t;
                    row_of_slot[t * k + s] = row;
                    dropped[t * k + s] = 0;
                } else {
                    row_of_slot[t * k + s] = -1;
                    dropped[t * k + s] = 1;
                }
                ++rank;
            }
    }
}

static double orc_act(int act, double a1, double a3)
{
    switch (act) {
    case ORC_ACT_RELU:
        return a1 > 0.0 ? a1 : 0.0;
    case ORC_ACT_GELU:
        /* exact GELU: a * Phi(a), Phi the standard normal CDF */
        return 0.5 * a1 * (1.0 + erf(a1 / sqrt(2.0)));
    default:
        /* SwiGLU ("Implementation": w2(silu(w1 x) * w3 x)), silu(z) = z / (1 + e^-z) */
        return (a1 / (1.0 + exp(-a1))) * a3;
    }
}

/*
 * Expert FFN on n (token, expert) pairs ("Implementation": the SwiGLU
 * expert w2(silu(w1 x) * w3 x) with bias-free Linears; ReLU and GELU
 * experts are d -> d_ff -> d with the activation between).
 *   tok, ex  [n]            token and expert of each pair
 *   x        [T][d]         fp32
 *   W1, W3   [E][d_ff][d]   fp32 (W3 only for SwiGLU, else may be NULL)
 *   W2       [E][d][d_ff]   fp32
 *   S1, S3   [E][d_ff]      fp32 per-row weight scales, or NULL (scale 1)
 *   S2       [E][d]         fp32 per-row weight scales, or NULL
 *   out      [n][d]         fp32: out[r] = fl32(W2_e fl32(act(W1_e x, W3_e x)))
 * Returns 0, or -1 when a thread's scratch cannot be allocated (then out is
 * incomplete and must not be used).
 * With scales, weight row i of a matrix is scale[i] times its stored row
 * (a row-scaled quantised matrix, orc_quantize_e4m3): each row's product
 * with the input is summed from the stored values and multiplied by the
 * scale once, in double, which equals the product with the scaled row.
 */
int orc_expert_ffn(int64_t n, const int32_t *tok, const int32_t *ex,
                   int64_t d, int64_t d_ff, int act, const float *x,
                   const float *W1, const float *W3, const float *W2,
                   const float *S1, const float *S3, const float *S2,
                   float *out)
{
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
    /* per-thread scratch: the hidden row and the widened input row */
    float *H = (float *)malloc((size_t)d_ff * sizeof(float));
    double *xd = (double *)malloc((size_t)(d > d_ff ? d : d_ff) * sizeof(double));
    if (!H || !xd)
        bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        if (!H || !xd)
            continue;   /* reported through the return value */
        const float *xr = x + (int64_t)tok[r] * d;
        const int64_t e = ex[r];
        const float *w1 = W1 + e * d_ff * d;
        const float *w3 = (act == ORC_ACT_SWIGLU) ? W3 + e * d_ff * d : NULL;
        const float *w2 = W2 + e * d * d_ff;
        for (int64_t j = 0; j < d; ++j)
            xd[j] = (double)xr[j];
        /* hidden: H_f = fl32(act(sum_j x_j W1[f][j], sum_j x_j W3[f][j])) */
        for (int64_t f0 = 0; f0 < d_ff; f0 += ORC_BLK) {
            int64_t nb = d_ff - f0 < ORC_BLK ? d_ff - f0 : ORC_BLK;
            double a1[ORC_BLK] = {0}, a3[ORC_BLK] = {0};
            for (int64_t j = 0; j < d; ++j)
                for (int64_t u = 0; u < nb; ++u)
                    a1[u] += xd[j] * (double)w1[(f0 + u) * d + j];
            if (w3)
                for (int64_t j = 0; j < d; ++j)
                    for (int64_t u = 0; u < nb; ++u)
                        a3[u] += xd[j] * (double)w3[(f0 + u) * d + j];
            if (S1)
                for (int64_t u = 0; u < nb; ++u)
                    a1[u] *= (double)S1[e * d_ff + f0 + u];
            if (w3 && S3)
                for (int64_t u = 0; u < nb; ++u)
                    a3[u] *= (double)S3[e * d_ff + f0 + u];
            for (int64_t u = 0; u < nb; ++u)
                H[f0 + u] = (float)orc_act(act, a1[u], a3[u]);
        }
        /* output: out_o = fl32(sum_f H_f W2[o][f]) */
        for (int64_t f = 0; f < d_ff; ++f)
            xd[f] = (double)H[f];
        for (int64_t o0 = 0; o0 < d; o0 += ORC_BLK) {
            int64_t nb = d - o0 < ORC_BLK ? d - o0 : ORC_BLK;
            double acc[ORC_BLK] = {0};
            for (int64_t f = 0; f < d_ff; ++f)
                for (int64_t u = 0; u < nb; ++u)
                    acc[u] += xd[f] * (double)w2[(o0 + u) * d_ff + f];
            for (int64_t u = 0; u < nb; ++u)
                out[r * d + o0 + u] = (float)(S2 ? acc[u] * (double)S2[e * d + o0 + u] : acc[u]);
        }
    }
    free(H);
    free(xd);
    }
    return bad ? -1 : 0;
}

/*
 * Gate-weighted combine ("Replacing the feed-forward block":
 * y = sum over the selected experts of g_i E_i(x); the Implementation
 * listing's index_add_ of the gated expert outputs).  Slots are summed in
 * slot order; a dropped slot contributes nothing, so a token whose every
 * slot was dropped gets 0 ("Capacity and dropped tokens": the residual,
 * outside the layer, carries it).
 *   gates [n][k] double
 *   rows  [n][k] int32: row of ys holding E_{idx[t][s]}(x_t), or -1 if dropped
 *   ys    [*][d] fp32 expert outputs
 *   y     [n][d] fp32 out
 */
void orc_combine(int64_t n, int64_t k, int64_t d, const double *gates,
                 const int32_t *rows, const float *ys, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t)
        for (int64_t o = 0; o < d; ++o) {
            double acc = 0.0;
            for (int64_t s = 0; s < k; ++s) {
                int32_t r = rows[t * k + s];
                if (r >= 0)
                    acc += gates[t * k + s] * (double)ys[(int64_t)r * d + o];
            }
            y[t * d + o] = (float)acc;
        }
}

/*
 * Layer output with shared experts and the block's residual.
 * Section "Total versus active parameters" names DeepSeek-V3's layer:
 * many small routed experts beside shared experts that every token visits.
 * The Implementation section's block adds the layer's output to its
 * hidden state, h + moe_out.  "Capacity and dropped tokens": a dropped
 * assignment skips its routed expert only; the residual still carries
 * the token, and (reading) so do the shared experts, which no routing
 * decision touches.  A shared expert has no gate (weight 1).
 *   gates, rows, ys  as orc_combine (routed part)
 *   S                shared experts
 *   ysh  [S][n][d]   fp32: shared expert j on token t is row j*n + t
 *   res  [n][d]      fp32 residual, or NULL for none
 *   y    [n][d]      fp32 out:
 *     y[t] = fl32(res[t] + (sum over kept slots, in slot order, of g ys[row]
 *                           + sum over j, in order, of ysh[j][t]))
 */
void orc_combine_shared(int64_t n, int64_t k, int64_t d, int64_t S, const double *gates,
                        const int32_t *rows, const float *ys, const float *ysh,
                        const float *res, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t)
        for (int64_t o = 0; o < d; ++o) {
            double moe_out = 0.0;
            for (int64_t s = 0; s < k; ++s) {
                int32_t r = rows[t * k + s];
                if (r >= 0)
                    moe_out += gates[t * k + s] * (double)ys[(int64_t)r * d + o];
            }
            for (int64_t j = 0; j < S; ++j)
                moe_out += (double)ysh[(j * n + t) * d + o];
            double h = res ? (double)res[t * d + o] : 0.0;
            y[t * d + o] = (float)(h + moe_out);
        }
}

/*
 * Load-balancing statistics ("The load-balancing loss"; the listing's
 * f, aux and z).  Means run over all T tokens, dropped ones included.
 *   f[i]  = #{t : idx[t][0] == i} / T   (top choice, before any drop)
 *   P[i]  = sum_t p[t][i] / T
 *   aux   = E * sum_i f[i] P[i]         (unweighted; alpha is applied by the caller)
 *   z     = sum_t lse[t]^2 / T          (unweighted)
 */
void orc_stats(int64_t T, int64_t E, int64_t k, const int32_t *idx,
               const double *p, const double *lse, double *f, double *P,
               double *aux, double *z)
{
    for (int64_t i = 0; i < E; ++i) {
        f[i] = 0.0;
        P[i] = 0.0;
    }
    for (int64_t t = 0; t < T; ++t)
        f[idx[t * k]] += 1.0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < E; ++i)
            P[i] += p[t * E + i];
    double a = 0.0, zz = 0.0;
    for (int64_t i = 0; i < E; ++i) {
        f[i] /= (double)T;
        P[i] /= (double)T;
        a += f[i] * P[i];
    }
    for (int64_t t = 0; t < T; ++t)
        zz += lse[t] * lse[t];
    *aux = (double)E * a;
    *z = zz / (double)T;
}

/*
 * 8-bit floating point E4M3 as the Open Compute Project's 8-bit floating
 * point specification (OFP8) defines it: a sign bit, 4 exponent bits with
 * bias 7 and 3 mantissa bits; exponent field 0 holds the subnormals
 * m/8 * 2^-6; the code with every exponent and mantissa bit set (0x7F,
 * 0xFF) is NaN, and there are no infinities, so the largest finite value
 * is 1.75 * 2^8 = 448.  The page "Mixture of experts" (rayaq.ca) finds
 * decoding limited by reading expert weights (Mechanics, "Total versus
 * active parameters") and names quantisation as a help to serving
 * ("Tradeoffs"); the glossary page "Mixture of Experts (MoE)" (inferensys.com,
 * inference optimization), in its entry on model quantization, describes
 * post-training quantisation of a trained model's weights to 8 bits.  The
 * format, the per-row scale and the rounding are readings: 8-bit weights in
 * the e4m3 format that gfx950's conversion units implement.
 */
double orc_e4m3_value(uint8_t c)
{
    const int sgn = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    if (ex == 15 && m == 7)
        return NAN;
    const double mag = ex == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, ex - 7);
    return sgn ? -mag : mag;
}

/*
 * The e4m3 code nearest to v (round to nearest, a tie to the code whose
 * mantissa is even); magnitudes beyond 448 give 448.  The sign of v (also
 * of a zero or of a value that rounds to zero) is kept.  Finite v only.
 * Positive codes 0x00..0x7E increase with their value, so the nearest one
 * is the last code not above |v| (found by bisection) or the code after it.
 */
uint8_t orc_e4m3_encode(float v)
{
    const double a = fabs((double)v);
    const uint8_t sgn = signbit(v) ? 0x80 : 0x00;
    int lo = 0, hi = 0x7F; /* value(lo) <= a, and hi is past the last candidate */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    int best = lo;
    if (lo < 0x7E) {
        const double dl = a - orc_e4m3_value((uint8_t)lo);
        const double dh = orc_e4m3_value((uint8_t)(lo + 1)) - a;
        if (dh < dl || (dh == dl && ((lo + 1) & 1) == 0))
            best = lo + 1;
    }
    return (uint8_t)(sgn | best);
}

/*
 * Post-training quantisation of a matrix, row by row (the model
 * quantization entry of the inference-optimization glossary page: reduced
 * precision weights, applied directly to a trained model): for each row i
 * of W [rows][cols],
 *   amax = max_j |W[i][j]|,  s[i] = fl32(amax / 448)  (1 if that is 0),
 *   q[i][j] = e4m3(clamp(fl32(W[i][j] / s[i]), -448, 448)),
 * every division a single fp32 division, so that the largest magnitude of
 * the row lands on +-448.  Row i of the matrix is then s[i] times the values
 * of its codes.
 */
void orc_quantize_e4m3(int64_t rows, int64_t cols, const float *W, uint8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *w = W + i * cols;
        float amax = 0.0f;
        for (int64_t j = 0; j < cols; ++j)
            if (fabsf(w[j]) > amax)
                amax = fabsf(w[j]);
        float si = amax / 448.0f;
        if (si == 0.0f)
            si = 1.0f;
        s[i] = si;
        for (int64_t j = 0; j < cols; ++j) {
            float v = w[j] / si;
            if (v > 448.0f)
                v = 448.0f;
            if (v < -448.0f)
                v = -448.0f;
            q[i * cols + j] = orc_e4m3_encode(v);
        }
    }
}

/* The values of n e4m3 codes, as fp32 (every finite code is exact in fp32). */
void orc_e4m3_decode(int64_t n, const uint8_t *q, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)orc_e4m3_value(q[i]);
}

/*
 * Backward of the layer (training): the gradients of
 *   L = sum_t <dy_t, y_t> + alpha_aux * aux + alpha_z * z
 * with respect to x, W_r, the router bias and the expert weights, for the
 * routing the forward took (the top-k choices and the capacity drops are
 * discrete, so they are held fixed; "Replacing the feed-forward block": the
 * router learns through the gate values, which are differentiable).
 *   - combine: y_t = sum over kept slots of g_ts E_e(x_t), so dE_e(x_t) =
 *     g_ts dy_t and dg_ts = <dy_t, E_e(x_t)> (0 for a dropped slot);
 *   - expert: a1 = W1 x, a3 = W3 x, H = act(a1, a3), E = W2 H (H stored in
 *     fp32 as in the forward); dH = W2^T dE, then through the activation
 *     (SwiGLU: H = silu(a1) a3, silu' = s (1 + a1 (1 - s)), s the logistic
 *     function; GELU: (a Phi(a))' = Phi(a) + a phi(a); ReLU: 1 for a > 0);
 *     dx += W1^T da1 + W3^T da3, dW1 += da1 x^T, dW3 += da3 x^T,
 *     dW2 += dE H^T, summed over the expert's kept rows in token order;
 *   - gates ("Top-k gating"): renormalised g = softmax of the selected
 *     logits, dh_sel = g (dg - <g, dg>); Switch g = p of the selected
 *     experts, dp = dg at those experts, dh = p (dp - <p, dp>);
 *   - "The load-balancing loss": aux = E sum_i f_i P_i with f_i the share of
 *     top choices (a count, constant) and P_i = mean_t p_ti, so
 *     d aux / d P_i = E f_i and dh_t += alpha_aux p_t (a - <p_t, a>) with
 *     a_i = E f_i / T; z = mean_t lse_t^2, so dh_t += alpha_z (2 / T) lse_t p_t;
 *   - router: h = W_r x + b + n, so dW_r = sum_t dh_t x_t^T, db = sum_t dh_t,
 *     dx_t += W_r^T dh_t.
 * Every sum in double, in index order; outputs rounded to fp32 once.
 *   rows [T][k]: row of slot (t, s) in the forward's permutation, -1 if
 *   dropped (only its sign is used here).  dbias may be NULL.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int orc_backward(int64_t T, int64_t d, int64_t d_ff, int64_t E, int64_t k, int gate, int act,
                 const float *x, const float *Wr, const float *bias, const float *noise,
                 const float *W1, const float *W3, const float *W2, const int32_t *rows,
                 const float *dy, double alpha_aux, double alpha_z, float *dx, float *dWr,
                 float *dbias, float *dW1, float *dW3, float *dW2)
{
    const int swiglu = act == ORC_ACT_SWIGLU;
    float *h = (float *)malloc((size_t)(T * E) * sizeof(float));
    int32_t *idx = (int32_t *)malloc((size_t)(T * k) * sizeof(int32_t));
    double *g = (double *)malloc((size_t)(T * k) * sizeof(double));
    double *p = (double *)malloc((size_t)(T * E) * sizeof(double));
    double *lse = (double *)malloc((size_t)T * sizeof(double));
    double *dg = (double *)calloc((size_t)(T * k), sizeof(double));
    double *dh = (double *)calloc((size_t)(T * E), sizeof(double));
    double *dxd = (double *)calloc((size_t)(T * d), sizeof(double));
    /* per kept slot: da1, da3, H (fp32 values) and dE */
    int64_t *pair_of = (int64_t *)malloc((size_t)(T * k) * sizeof(int64_t));
    int rc = -1;
    if (!h || !idx || !g || !p || !lse || !dg || !dh || !dxd || !pair_of)
        goto out;
    orc_router_logits(T, d, E, x, Wr, bias, noise, h);
    if (orc_gate(T, E, k, gate, h, idx, g, p, lse) != 0)
        goto out;
    int64_t n = 0;
    for (int64_t i = 0; i < T * k; ++i)
        pair_of[i] = rows[i] >= 0 ? n++ : -1;
    {
        double *da1 = (double *)calloc((size_t)(n * d_ff) + 1, sizeof(double));
        double *da3 = (double *)calloc((size_t)(n * d_ff) + 1, sizeof(double));
        double *Hs = (double *)calloc((size_t)(n * d_ff) + 1, sizeof(double));
        double *dE = (double *)calloc((size_t)(n * d) + 1, sizeof(double));
        if (!da1 || !da3 || !Hs || !dE) {
            free(da1);
            free(da3);
            free(Hs);
            free(dE);
            goto out;
        }
        /* expert part, one token at a time */
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            const float *xt = x + t * d;
            for (int64_t s = 0; s < k; ++s) {
                const int64_t q = pair_of[t * k + s];
                if (q < 0)
                    continue;
                const int64_t e = idx[t * k + s];
                const float *w1 = W1 + e * d_ff * d, *w3 = swiglu ? W3 + e * d_ff * d : NULL;
                const float *w2 = W2 + e * d * d_ff;
                double *a1 = da1 + q * d_ff, *a3 = da3 + q * d_ff, *Hq = Hs + q * d_ff;
                for (int64_t f = 0; f < d_ff; ++f) {
                    double u = 0.0, v = 0.0;
                    for (int64_t j = 0; j < d; ++j) {
                        u += (double)xt[j] * (double)w1[f * d + j];
                        if (w3)
                            v += (double)xt[j] * (double)w3[f * d + j];
                    }
                    a1[f] = u; /* pre-activations for now */
                    a3[f] = v;
                    Hq[f] = (double)(float)orc_act(act, u, v);
                }
                /* E(x_t) (stored fp32 in the forward), dg and dE */
                double dgs = 0.0;
                for (int64_t o = 0; o < d; ++o) {
                    double acc = 0.0;
                    for (int64_t f = 0; f < d_ff; ++f)
                        acc += Hq[f] * (double)w2[o * d_ff + f];
                    dgs += (double)dy[t * d + o] * (double)(float)acc;
                    dE[q * d + o] = g[t * k + s] * (double)dy[t * d + o];
                }
                dg[t * k + s] = dgs;
                /* dH = W2^T dE, then the activation's derivative */
                for (int64_t f = 0; f < d_ff; ++f) {
                    double dH = 0.0;
                    for (int64_t o = 0; o < d; ++o)
                        dH += (double)w2[o * d_ff + f] * dE[q * d + o];
                    const double u = a1[f], v = a3[f];
                    if (act == ORC_ACT_SWIGLU) {
                        const double sg = 1.0 / (1.0 + exp(-u));
                        a1[f] = dH * v * sg * (1.0 + u * (1.0 - sg));
                        a3[f] = dH * u * sg;
                    } else if (act == ORC_ACT_GELU) {
                        const double Phi = 0.5 * (1.0 + erf(u / sqrt(2.0)));
                        const double phi = exp(-0.5 * u * u) / sqrt(2.0 * acos(-1.0)); /* normal density */
                        a1[f] = dH * (Phi + u * phi);
                        a3[f] = 0.0;
                    } else {
                        a1[f] = u > 0.0 ? dH : 0.0;
                        a3[f] = 0.0;
                    }
                }
                /* dx_t += W1^T da1 + W3^T da3 */
                for (int64_t j = 0; j < d; ++j) {
                    double acc = 0.0;
                    for (int64_t f = 0; f < d_ff; ++f) {
                        acc += a1[f] * (double)w1[f * d + j];
                        if (w3)
                            acc += a3[f] * (double)w3[f * d + j];
                    }
                    dxd[t * d + j] += acc;
                }
            }
        }
        /* weight gradients: per expert row, the kept rows in token order */
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t ef = 0; ef < E * d_ff; ++ef) {
            const int64_t e = ef / d_ff, f = ef - e * d_ff;
            double *acc1 = (double *)calloc((size_t)d, sizeof(double));
            double *acc3 = (double *)calloc((size_t)d, sizeof(double));
            if (!acc1 || !acc3) {
                free(acc1);
                free(acc3);
                continue;
            }
            for (int64_t t = 0; t < T; ++t)
                for (int64_t s = 0; s < k; ++s) {
                    const int64_t q = pair_of[t * k + s];
                    if (q < 0 || idx[t * k + s] != e)
                        continue;
                    for (int64_t j = 0; j < d; ++j) {
                        acc1[j] += da1[q * d_ff + f] * (double)x[t * d + j];
                        acc3[j] += da3[q * d_ff + f] * (double)x[t * d + j];
                    }
                }
            for (int64_t j = 0; j < d; ++j) {
                dW1[(e * d_ff + f) * d + j] = (float)acc1[j];
                if (swiglu)
                    dW3[(e * d_ff + f) * d + j] = (float)acc3[j];
            }
            free(acc1);
            free(acc3);
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t eo = 0; eo < E * d; ++eo) {
            const int64_t e = eo / d, o = eo - e * d;
            double *acc = (double *)calloc((size_t)d_ff, sizeof(double));
            if (!acc)
                continue;
            for (int64_t t = 0; t < T; ++t)
                for (int64_t s = 0; s < k; ++s) {
                    const int64_t q = pair_of[t * k + s];
                    if (q < 0 || idx[t * k + s] != e)
                        continue;
                    for (int64_t f = 0; f < d_ff; ++f)
                        acc[f] += dE[q * d + o] * Hs[q * d_ff + f];
                }
            for (int64_t f = 0; f < d_ff; ++f)
                dW2[(e * d + o) * d_ff + f] = (float)acc[f];
            free(acc);
        }
        free(da1);
        free(da3);
        free(Hs);
        free(dE);
    }
    /* router: gates, then the statistics' terms */
    {
        double *fsh = (double *)calloc((size_t)E, sizeof(double));
        if (!fsh)
            goto out;
        for (int64_t t = 0; t < T; ++t)
            fsh[idx[t * k]] += 1.0;
        for (int64_t i = 0; i < E; ++i)
            fsh[i] /= (double)T;
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double *pt = p + t * E;
            double *dht = dh + t * E;
            if (gate == ORC_GATE_RENORM) {
                double dot = 0.0;
                for (int64_t s = 0; s < k; ++s)
                    dot += g[t * k + s] * dg[t * k + s];
                for (int64_t s = 0; s < k; ++s)
                    dht[idx[t * k + s]] += g[t * k + s] * (dg[t * k + s] - dot);
            } else {
                double dot = 0.0;
                for (int64_t s = 0; s < k; ++s)
                    dot += pt[idx[t * k + s]] * dg[t * k + s];
                for (int64_t i = 0; i < E; ++i)
                    dht[i] -= pt[i] * dot;
                for (int64_t s = 0; s < k; ++s)
                    dht[idx[t * k + s]] += pt[idx[t * k + s]] * dg[t * k + s];
            }
            if (alpha_aux != 0.0) {
                double dot = 0.0;
                for (int64_t i = 0; i < E; ++i)
                    dot += pt[i] * ((double)E * fsh[i] / (double)T);
                for (int64_t i = 0; i < E; ++i)
                    dht[i] += alpha_aux * pt[i] * ((double)E * fsh[i] / (double)T - dot);
            }
            if (alpha_z != 0.0)
                for (int64_t i = 0; i < E; ++i)
                    dht[i] += alpha_z * 2.0 / (double)T * lse[t] * pt[i];
            for (int64_t j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < E; ++i)
                    acc += dht[i] * (double)Wr[i * d + j];
                dxd[t * d + j] += acc;
            }
        }
        free(fsh);
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < E; ++i) {
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += dh[t * E + i] * (double)x[t * d + j];
            dWr[i * d + j] = (float)acc;
        }
        if (dbias) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += dh[t * E + i];
            dbias[i] = (float)acc;
        }
    }
    for (int64_t i = 0; i < T * d; ++i)
        dx[i] = (float)dxd[i];
    rc = 0;
out:
    free(h);
    free(idx);
    free(g);
    free(p);
    free(lse);
    free(dg);
    free(dh);
    free(dxd);
    free(pair_of);
    return rc;
}

/*
 * Weight gradients of ONE expert for selected hidden units only (the
 * layer's backward of orc_backward restricted to what a sample of a large
 * layer needs): for every f in fsel, row f of dW1 and dW3 and column f of
 * dW2, from the expert's kept rows in token order (page "Mixture of
 * experts", Mechanics: the gate multiplies the expert output; the expert is
 * the Implementation section's w2(act(w1 x) [* w3 x])).  For each kept row
 * r (token t_r, gate g_r):
 *   dE_r      = g_r * dy[t_r]                        (gradient of the expert output)
 *   a1, a3    = W1[f] . x[t_r],  W3[f] . x[t_r]      (double)
 *   H_r       = fl32(act(a1, a3))                    (the forward's stored hidden unit)
 *   dH_r      = sum_o W2[o][f] dE_r[o]
 *   da1, da3  = the activation's derivative times dH_r
 * and, summed over the rows in order and rounded once,
 *   dW1s[i][j] = sum_r da1_r x[t_r][j],  dW3s[i][j] = sum_r da3_r x[t_r][j],
 *   dW2s[o][i] = sum_r dE_r[o] H_r          (f = fsel[i]).
 *   tok, gate  [n]        kept rows of the expert: token and gate
 *   W1, W3     [d_ff][d]  this expert's up projections (W3 only for SwiGLU)
 *   W2         [d][d_ff]  this expert's down projection
 *   dy         [T][d], x [T][d]
 *   dW1s, dW3s [nf][d];  dW2s [d][nf]
 * Returns 0, or -1 when scratch cannot be allocated.
 */
int orc_expert_wgrad_sel(int64_t n, const int32_t *tok, const double *gate, int64_t d, int64_t d_ff,
                         int act, const float *x, const float *W1, const float *W3, const float *W2,
                         const float *dy, int64_t nf, const int32_t *fsel, float *dW1s, float *dW3s,
                         float *dW2s)
{
    const int swiglu = act == ORC_ACT_SWIGLU;
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
    double *da1 = (double *)malloc((size_t)(n + 1) * sizeof(double));
    double *da3 = (double *)malloc((size_t)(n + 1) * sizeof(double));
    double *Hr = (double *)malloc((size_t)(n + 1) * sizeof(double));
    if (!da1 || !da3 || !Hr)
        bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nf; ++i) {
        if (!da1 || !da3 || !Hr)
            continue;
        const int64_t f = fsel[i];
        const float *w1 = W1 + f * d, *w3 = swiglu ? W3 + f * d : NULL;
        for (int64_t r = 0; r < n; ++r) {
            const float *xt = x + (int64_t)tok[r] * d;
            const float *dyt = dy + (int64_t)tok[r] * d;
            double u = 0.0, v = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                u += (double)xt[j] * (double)w1[j];
                if (w3)
                    v += (double)xt[j] * (double)w3[j];
            }
            Hr[r] = (double)(float)orc_act(act, u, v);
            double dH = 0.0;
            for (int64_t o = 0; o < d; ++o)
                dH += (double)W2[o * d_ff + f] * (gate[r] * (double)dyt[o]);
            if (act == ORC_ACT_SWIGLU) {
                const double sg = 1.0 / (1.0 + exp(-u));
                da1[r] = dH * v * sg * (1.0 + u * (1.0 - sg));
                da3[r] = dH * u * sg;
            } else if (act == ORC_ACT_GELU) {
                const double Phi = 0.5 * (1.0 + erf(u / sqrt(2.0)));
                const double phi = exp(-0.5 * u * u) / sqrt(2.0 * acos(-1.0));
                da1[r] = dH * (Phi + u * phi);
                da3[r] = 0.0;
            } else {
                da1[r] = u > 0.0 ? dH : 0.0;
                da3[r] = 0.0;
            }
        }
        for (int64_t j = 0; j < d; ++j) {
            double a = 0.0, b = 0.0;
            for (int64_t r = 0; r < n; ++r) {
                const double xv = (double)x[(int64_t)tok[r] * d + j];
                a += da1[r] * xv;
                b += da3[r] * xv;
            }
            dW1s[i * d + j] = (float)a;
            if (swiglu)
                dW3s[i * d + j] = (float)b;
        }
        for (int64_t o = 0; o < d; ++o) {
            double a = 0.0;
            for (int64_t r = 0; r < n; ++r)
                a += (gate[r] * (double)dy[(int64_t)tok[r] * d + o]) * Hr[r];
            dW2s[o * nf + i] = (float)a;
        }
    }
    free(da1);
    free(da3);
    free(Hr);
    }
    return bad ? -1 : 0;
}

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of host threads the oracle's parallel loops use. */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets that number (n >= 1); results do not depend on it, since threads
 * split tokens and rows, never a sum. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
