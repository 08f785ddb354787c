/*
 * oracle.c -- plain, slow, sequential fp64 reference for the GDN core.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): never linked into, loaded by or
 * called from the product path.  Scalar loops, libm exp/sqrt, no SIMD, no
 * blocking, no fast-math; built with -ffp-contract=off so every rounding is
 * the one written here.
 *
 * Page tags as in oracle.h: [P1] RL-Kernel PR #469 (GDN decode-step goldens
 * and recurrent/conv state contract), [P4] vLLM PR #53864 (CuteDSL GDN
 * prefill).  Readings of points the pages leave open are listed beside the
 * code that takes them.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Index validation ([P1] "State ABI": the goldens raise on an active index   */
/* that is out of range or repeated; indices <= 0 are inactive).             */
/* ------------------------------------------------------------------------- */
static int check_slots(const int32_t* slot_idx, int32_t n, int32_t num_slots)
{
    int err = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t s = slot_idx[i];
        if (s <= 0) continue;                 /* inactive row */
        if (s >= num_slots) err |= ORACLE_ERR_SLOT_RANGE;
        for (int32_t j = 0; j < i; ++j)
            if (slot_idx[j] == s) err |= ORACLE_ERR_SLOT_REPEAT;
    }
    return err;
}

static int check_seqlens(const int32_t* cu, int32_t n_seqs, int64_t total)
{
    if (cu[0] != 0) return ORACLE_ERR_SEQLENS;
    for (int32_t i = 0; i < n_seqs; ++i)
        if (cu[i + 1] < cu[i]) return ORACLE_ERR_SEQLENS;
    if ((int64_t)cu[n_seqs] != total) return ORACLE_ERR_SEQLENS;
    return 0;
}

/* SiLU, y * sigmoid(y) = y / (1 + exp(-y))  ([P1] "The conv half"). */
static double silu(double y) { return y / (1.0 + exp(-y)); }

/* ------------------------------------------------------------------------- */
/* Causal conv1d over one run of tokens of one sequence.                      */
/* X = [state[c, 0..W-2], x_0[c], ..., x_{L-1}[c]] (oldest first);            */
/* y_t[c] = bias[c] + sum_j weight[c, j] * X[t + j]  (bias-first accumulator, */
/* [P1] "Summary", conv half); the new state is the last W-1 entries of X,    */
/* copied unchanged.  Reading: tap j = W-1 multiplies the current token (a    */
/* standard causal convolution; the pages do not print the tap order).        */
/* ------------------------------------------------------------------------- */
static void conv_run(const double* x, int64_t L, double* state,
                     const double* weight, const double* bias, double* out,
                     int32_t dim, int32_t width, int32_t flags)
{
    const int32_t W1 = width - 1;
    double* X = (double*)malloc(sizeof(double) * (size_t)(W1 + L));
    for (int32_t c = 0; c < dim; ++c) {
        for (int32_t j = 0; j < W1; ++j) X[j] = state[(size_t)c * W1 + j];
        for (int64_t t = 0; t < L; ++t) X[W1 + t] = x[(size_t)t * dim + c];
        for (int64_t t = 0; t < L; ++t) {
            double y = bias ? bias[c] : 0.0;
            for (int32_t j = 0; j < width; ++j)
                y += weight[(size_t)c * width + j] * X[t + j];
            if (flags & ORACLE_FLAG_SILU) y = silu(y);
            out[(size_t)t * dim + c] = y;
        }
        for (int32_t j = 0; j < W1; ++j)
            state[(size_t)c * W1 + j] = X[L + j];
    }
    free(X);
}

int oracle_conv_update(const double* x, int64_t total_tokens,
                       const int32_t* cu_seqlens, int32_t n_seqs,
                       const int32_t* slot_idx,
                       double* conv_state, int32_t num_slots,
                       const double* weight, const double* bias,
                       double* out, int32_t dim, int32_t width, int32_t flags)
{
    if (n_seqs < 0 || dim <= 0 || width < 1 || num_slots < 1 || total_tokens < 0)
        return ORACLE_ERR_ARGS;
    if (!cu_seqlens && total_tokens != n_seqs) return ORACLE_ERR_ARGS;
    int err = check_slots(slot_idx, n_seqs, num_slots);
    if (cu_seqlens) err |= check_seqlens(cu_seqlens, n_seqs, total_tokens);
    if (err) return err;

    const size_t state_sz = (size_t)dim * (size_t)(width - 1);
    for (int32_t n = 0; n < n_seqs; ++n) {
        int64_t start = cu_seqlens ? cu_seqlens[n] : n;
        int64_t L = cu_seqlens ? (int64_t)cu_seqlens[n + 1] - cu_seqlens[n] : 1;
        int32_t s = slot_idx[n];
        if (s <= 0) {                     /* inactive: zero output, no cache access */
            memset(out + (size_t)start * dim, 0, sizeof(double) * (size_t)L * dim);
            continue;
        }
        if (L == 0) continue;             /* reading: empty run leaves the state alone */
        conv_run(x + (size_t)start * dim, L, conv_state + (size_t)s * state_sz,
                 weight, bias, out + (size_t)start * dim, dim, width, flags);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* One token of the gated delta rule on one value head's state S[dv][dk].     */
/*   alpha = exp(g); S1 = alpha * S; u = S1 k; S' = S1 + beta (v - u) k^T;    */
/*   o = S' q.                                                                */
/* Expanding S' gives exactly exp(g) S (I - beta k k^T) + beta v k^T.  The    */
/* decay is applied before the prediction S k (u uses the decayed state).     */
/* ------------------------------------------------------------------------- */
static void delta_rule_token(double* S, const double* q, const double* k,
                             const double* v, double g, double beta,
                             double* o, int32_t dk, int32_t dv)
{
    const double alpha = exp(g);
    for (int32_t i = 0; i < dv; ++i) {
        double* row = S + (size_t)i * dk;
        for (int32_t j = 0; j < dk; ++j) row[j] = alpha * row[j];
        double u = 0.0;
        for (int32_t j = 0; j < dk; ++j) u += row[j] * k[j];
        const double delta = beta * (v[i] - u);
        for (int32_t j = 0; j < dk; ++j) row[j] = row[j] + delta * k[j];
        double acc = 0.0;
        for (int32_t j = 0; j < dk; ++j) acc += row[j] * q[j];
        o[i] = acc;
    }
}

/* q/k L2 norm x / sqrt(sum(x*x) + 1e-6), then q times scale; k is never scaled
   ([P1] "How the golden relates to the kernel", item 3).  When the norm flag
   is off only the scale is applied to q. */
static void prepare_qk(const double* qin, const double* kin, double* q, double* k,
                       int32_t dk, double scale, int32_t flags)
{
    double qn = 1.0, kn = 1.0;
    if (flags & ORACLE_FLAG_QK_L2NORM) {
        double sq = 0.0, sk = 0.0;
        for (int32_t j = 0; j < dk; ++j) { sq += qin[j] * qin[j]; sk += kin[j] * kin[j]; }
        qn = 1.0 / sqrt(sq + 1e-6);
        kn = 1.0 / sqrt(sk + 1e-6);
    }
    for (int32_t j = 0; j < dk; ++j) {
        q[j] = qin[j] * qn * scale;
        k[j] = kin[j] * kn;
    }
}

int oracle_decode_step(const double* mixed_qkv, const double* g, const double* beta,
                       const int32_t* slot_idx, int32_t batch,
                       double* conv_state, const double* conv_weight,
                       const double* conv_bias,
                       double* rec_state, int32_t num_slots, double* out,
                       int32_t H, int32_t HV, int32_t dk, int32_t dv, int32_t W,
                       double scale, int32_t flags)
{
    if (batch < 0 || H <= 0 || HV <= 0 || HV % H != 0 || dk <= 0 || dv <= 0 ||
        W < 1 || num_slots < 1)
        return ORACLE_ERR_ARGS;
    int err = check_slots(slot_idx, batch, num_slots);
    if (err) return err;

    const int32_t D = 2 * H * dk + HV * dv;
    const int32_t group = HV / H;       /* value heads per key head */
    const size_t cs_sz = (size_t)D * (size_t)(W - 1);
    const size_t rs_sz = (size_t)HV * dv * dk;
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    double* q = (double*)malloc(sizeof(double) * (size_t)dk);
    double* k = (double*)malloc(sizeof(double) * (size_t)dk);

    for (int32_t b = 0; b < batch; ++b) {
        double* ob = out + (size_t)b * HV * dv;
        int32_t s = slot_idx[b];
        if (s <= 0) {                        /* [P1] "State ABI": zeros, untouched */
            memset(ob, 0, sizeof(double) * (size_t)HV * dv);
            continue;
        }
        /* conv over the single new token, then SiLU */
        conv_run(mixed_qkv + (size_t)b * D, 1, conv_state + (size_t)s * cs_sz,
                 conv_weight, conv_bias, y, D, W, flags);
        /* split [q | k | v], head-major; GQA map h = hv / (HV / H)
           ([P1] "How the golden relates", item 2) */
        for (int32_t hv = 0; hv < HV; ++hv) {
            const int32_t h = hv / group;
            prepare_qk(y + (size_t)h * dk, y + (size_t)H * dk + (size_t)h * dk, q, k,
                       dk, scale, flags);
            const double* v = y + (size_t)2 * H * dk + (size_t)hv * dv;
            delta_rule_token(rec_state + (size_t)s * rs_sz + (size_t)hv * dv * dk,
                             q, k, v, g[(size_t)b * HV + hv], beta[(size_t)b * HV + hv],
                             ob + (size_t)hv * dv, dk, dv);
        }
    }
    free(y); free(q); free(k);
    return 0;
}

int oracle_prefill(const double* qin, const double* kin, const double* vin,
                   const double* g, const double* beta,
                   const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                   const int32_t* slot_idx,
                   double* rec_state, int32_t num_slots, double* out,
                   int32_t H, int32_t HV, int32_t dk, int32_t dv,
                   double scale, int32_t flags)
{
    if (n_seqs < 0 || H <= 0 || HV <= 0 || HV % H != 0 || dk <= 0 || dv <= 0 ||
        num_slots < 1 || total_tokens < 0 || !cu_seqlens)
        return ORACLE_ERR_ARGS;
    int err = check_slots(slot_idx, n_seqs, num_slots);
    err |= check_seqlens(cu_seqlens, n_seqs, total_tokens);
    if (err) return err;

    const int32_t group = HV / H;
    const size_t rs_sz = (size_t)HV * dv * dk;
    double* q = (double*)malloc(sizeof(double) * (size_t)dk);
    double* k = (double*)malloc(sizeof(double) * (size_t)dk);

    for (int32_t n = 0; n < n_seqs; ++n) {
        const int64_t start = cu_seqlens[n], end = cu_seqlens[n + 1];
        const int32_t s = slot_idx[n];
        if (s <= 0) {
            memset(out + (size_t)start * HV * dv, 0,
                   sizeof(double) * (size_t)(end - start) * HV * dv);
            continue;
        }
        for (int32_t hv = 0; hv < HV; ++hv) {
            const int32_t h = hv / group;
            double* S = rec_state + (size_t)s * rs_sz + (size_t)hv * dv * dk;
            for (int64_t t = start; t < end; ++t) {
                prepare_qk(qin + ((size_t)t * H + h) * dk, kin + ((size_t)t * H + h) * dk,
                           q, k, dk, scale, flags);
                delta_rule_token(S, q, k, vin + ((size_t)t * HV + hv) * dv,
                                 g[(size_t)t * HV + hv], beta[(size_t)t * HV + hv],
                                 out + ((size_t)t * HV + hv) * dv, dk, dv);
            }
        }
    }
    free(q); free(k);
    return 0;
}

/* [P1] "How the golden relates to the kernel", item 1: fused fp32 gating with
 * the softplus threshold at 20.  Here in fp64; log1p keeps log(1 + e^x)
 * accurate where e^x is small. */
static double softplus_thresholded(double x)
{
    return (x <= 20.0) ? log1p(exp(x)) : x;
}

int oracle_gating(const double* a, const double* b, const double* A_log,
                  const double* dt_bias, int64_t rows, int32_t num_v_heads,
                  double* g, double* beta)
{
    if (rows < 0 || num_v_heads <= 0) return ORACLE_ERR_ARGS;
    if (rows > 0 && (!a || !b || !A_log || !dt_bias || !g || !beta)) return ORACLE_ERR_ARGS;
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t h = 0; h < num_v_heads; ++h) {
            const int64_t i = r * num_v_heads + h;
            g[i] = -exp(A_log[h]) * softplus_thresholded(a[i] + dt_bias[h]);
            beta[i] = 1.0 / (1.0 + exp(-b[i]));
        }
    }
    return 0;
}

/* Gated RMSNorm: the plain definition (norm first, then weight and gate). */
int oracle_gated_rmsnorm(const double* x, const double* z, const double* weight,
                         int64_t rows, int32_t dim, double eps, int32_t flags, double* out)
{
    if (rows < 0 || dim <= 0 || eps < 0.0) return ORACLE_ERR_ARGS;
    if (rows > 0 && (!x || !weight || !out)) return ORACLE_ERR_ARGS;
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * dim;
        double ss = 0.0;
        for (int32_t j = 0; j < dim; ++j) ss += xr[j] * xr[j];
        const double rms = sqrt(ss / dim + eps);
        for (int32_t j = 0; j < dim; ++j) {
            const double w = (flags & ORACLE_NORM_ZERO_CENTRED) ? weight[j] + 1.0 : weight[j];
            double gate = 1.0;
            if (z) {
                const double zj = z[r * dim + j];
                const double sig = 1.0 / (1.0 + exp(-zj));
                gate = (flags & ORACLE_NORM_GATE_SIGMOID) ? sig : zj * sig;
            }
            out[r * dim + j] = (rms > 0.0 ? xr[j] / rms : 0.0) * w * gate;
        }
    }
    return 0;
}
